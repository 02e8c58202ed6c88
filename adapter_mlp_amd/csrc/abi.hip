// C-ABI entry points: argument validation, workspace planning and the kernel
// sequence of each call.  Every check runs on the host before the first
// enqueue, so a call that returns an error has enqueued nothing.
#include <cmath>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>

#include "common.hpp"
#include "kernels.hpp"
#include "trace.hpp"

using namespace lora;

// Static scratch of lora_o_fwd_noalloc (see static_scratch below).
constexpr size_t kScratchBytes = LORA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error = "no error";

lora_status fail(lora_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lora_status fail(lora_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

#define CHECK(cond, status, ...)          \
  do {                                    \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define LAUNCH(expr)                                                              \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) return fail(LORA_EDEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// LAUNCH with the launch bracketed for lora_trace_* under `name`.
#define LAUNCHN(name, stream, expr)       \
  do {                                    \
    TraceScope ts_(name, stream);         \
    LAUNCH(expr);                         \
  } while (0)

inline int64_t pad16(int64_t x) { return (x + 15) / 16 * 16; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Ctx {
  bool bf16;
  bool f32lora;  // LORA_BF16_F32LORA: fp32 adapters and adapter gradients
  size_t es;     // element size of the activations and the base
  const lora_plan* plan = nullptr;  // the call's GEMM launch plan (bf16 only)
  // Width of the GEMM's LoRA K tile: one full 64-wide tile (zero-padded) in bf16.
  int64_t rl(int64_t w) const { return bf16 ? 64 : w; }
};

// Bump allocator over the caller's workspace (256-byte aligned pieces).
struct Ws {
  char* base;
  size_t off = 0;
  explicit Ws(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// `adapters` admits LORA_BF16_F32LORA (the calls that take adapters).
lora_status check_dtype(int32_t dtype, Ctx& c, bool adapters = false) {
  CHECK(dtype == LORA_F32 || dtype == LORA_BF16 || (adapters && dtype == LORA_BF16_F32LORA), LORA_EDTYPE,
        "unknown dtype %d", dtype);
  c.bf16 = dtype != LORA_F32;
  c.f32lora = dtype == LORA_BF16_F32LORA;
  c.es = c.bf16 ? 2 : 4;
  return LORA_OK;
}

lora_status check_dim(const Ctx& c, int64_t v, const char* name) {
  CHECK(v > 0, LORA_ESHAPE, "%s = %lld must be positive", name, (long long)v);
  if (c.bf16) CHECK(v % 64 == 0, LORA_ESHAPE, "%s = %lld must be a multiple of 64 for bf16", name, (long long)v);
  return LORA_OK;
}

lora_status check_rank(const Ctx& c, int64_t r, int group) {
  CHECK(r >= 1 && r <= 64, LORA_ESHAPE, "rank r = %lld must be in [1, 64]", (long long)r);
  if (c.bf16) {
    CHECK(r % 8 == 0, LORA_ESHAPE, "rank r = %lld must be a multiple of 8 for bf16", (long long)r);
    CHECK(r * group <= 64, LORA_ESHAPE, "adapter group width %lld exceeds 64", (long long)(r * group));
  }
  return LORA_OK;
}

// Kernels address each operand with 32-bit byte offsets.
lora_status check_extent(const Ctx& c, int64_t rows, int64_t cols, const char* what) {
  const int64_t lim = ((int64_t)1 << 31) - 4096;
  CHECK(rows <= lim / (cols * (int64_t)c.es), LORA_ESHAPE, "%s (%lld x %lld) exceeds 2 GiB", what,
        (long long)rows, (long long)cols);
  return LORA_OK;
}

lora_status check_ptr(const Ctx& c, const void* p, const char* name) {
  CHECK(p != nullptr, LORA_EINVAL, "%s is NULL", name);
  CHECK(aligned(p, c.bf16 ? 16 : 4), LORA_EALIGN, "%s is not %d-byte aligned", name, c.bf16 ? 16 : 4);
  return LORA_OK;
}

// A tensor with T rows may be NULL when T == 0 (an empty allocation).
lora_status check_tptr(const Ctx& c, const void* p, int64_t T, const char* name) {
  if (T == 0 && p == nullptr) return LORA_OK;
  return check_ptr(c, p, name);
}

#define TRY(expr)                    \
  do {                               \
    lora_status s_ = (expr);         \
    if (s_ != LORA_OK) return s_;    \
  } while (0)

lora_status check_nf4(const lora_nf4* q, int64_t rows, int64_t cols, const char* name) {
  CHECK(q->codes && q->q8 && q->s2 && q->mu, LORA_EINVAL, "%s: NF4 array pointer is NULL", name);
  CHECK(q->rows == rows && q->cols == cols, LORA_ESHAPE,
        "%s: NF4 weight is [%lld, %lld], expected [%lld, %lld]", name, (long long)q->rows,
        (long long)q->cols, (long long)rows, (long long)cols);
  CHECK((rows * cols) % NF4_GROUP == 0, LORA_ESHAPE, "%s: NF4 numel %lld not a multiple of %lld", name,
        (long long)(rows * cols), (long long)NF4_GROUP);
  CHECK(aligned(q->codes, 4) && aligned(q->s2, 4) && aligned(q->mu, 4), LORA_EALIGN,
        "%s: NF4 codes/s2/mu must be 4-byte aligned", name);
  return LORA_OK;
}

lora_status check_proj(const Ctx& c, const lora_proj* p, int64_t n_in, int64_t n_out, const char* name) {
  CHECK(p != nullptr, LORA_EINVAL, "%s is NULL", name);
  CHECK((p->W != nullptr) != (p->nf4 != nullptr), LORA_EINVAL, "%s: exactly one of W and nf4 must be set", name);
  if (p->nf4) {
    CHECK(c.bf16, LORA_EUNSUPPORTED, "%s: NF4 base needs the bf16 compute dtype", name);
    TRY(check_nf4(p->nf4, n_in, n_out, name));
  } else {
    TRY(check_ptr(c, p->W, name));
  }
  if (p->Wt) {
    CHECK(p->W != nullptr, LORA_EINVAL, "%s: Wt is only for a dense W", name);
    TRY(check_ptr(c, p->Wt, name));
  }
  TRY(check_ptr(c, p->A, name));
  TRY(check_ptr(c, p->B, name));
  CHECK(std::isfinite(p->scale), LORA_EINVAL, "%s: scale is not finite", name);
  return LORA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + nb && y < x + na;
}

BSrc bsrc(const lora_proj* p, int64_t ld) {
  BSrc s{};
  if (p->nf4) {
    s.codes = p->nf4->codes;
    s.q8 = p->nf4->q8;
    s.s2 = p->nf4->s2;
    s.mu = p->nf4->mu;
    s.wcols = p->nf4->cols;
  } else {
    s.p = p->W;
    s.ld = ld;
  }
  return s;
}

// A forward GEMM reads the K-contiguous copies Wt when every projection it
// reads has one (bf16): B_NT over Wt [n_out, n_in] (row pitch n_in).
bool fwd_t(const Ctx& c, std::initializer_list<const lora_proj*> ps) {
  if (!c.bf16) return false;
  for (const lora_proj* p : ps)
    if (p->Wt == nullptr) return false;
  return true;
}
BSrc bsrc_t(const lora_proj* p, int64_t n_in) {
  BSrc s{};
  s.p = p->Wt;
  s.ld = n_in;
  return s;
}

const void* coff(const void* p, int64_t elems, const Ctx& c) {
  return static_cast<const char*>(p) + elems * (int64_t)c.es;
}
void* offw(void* p, int64_t elems, const Ctx& c) { return static_cast<char*>(p) + elems * (int64_t)c.es; }

// Plan entry i of the call (zeros: the library's defaults; always zeros in fp32).
lora_gemm_plan gemm_plan(const Ctx& c, int i) {
  if (!c.bf16 || c.plan == nullptr) return lora_gemm_plan{0, 0};
  return c.plan->gemm[i];
}

// Split-K factor of a bf16 store GEMM [M, N] over K (LoRA tile included): the
// s in 1..4 that best fills the last wave of 256x256 tiles on the 256 CUs,
// weighed against the fp32 partials it writes and reads (8 s bytes per
// output element, about 1040 s / K of the GEMM's time at the measured GEMM
// and HBM rates).  Each part keeps at least 16 K steps of 64.
int gemm_ksplit(const Ctx& c, int64_t M, int64_t N, int64_t K) {
  if (!c.bf16) return 1;
  // each fp32 part [M, N] must stay below 2 GiB (32-bit offsets of its stores)
  if (M * N * 4 >= ((int64_t)1 << 31) - 4096) return 1;
  const int64_t tiles = cdiv(M, 256) * cdiv(N, 256);
  if (tiles == 0) return 1;
  double best = 0.0;
  int bs = 1;
  for (int s = 1; s <= 4; ++s) {
    if (s > 1 && K / 64 / s < 16) break;
    const int64_t units = tiles * s;
    const double fill = (double)units / (double)(cdiv(units, 256) * 256);
    const double score = fill / (s > 1 ? 1.0 + 1040.0 * s / (double)K : 1.0);
    if (score > best * 1.02) {
      best = score;
      bs = s;
    }
  }
  return bs;
}
// First split tile of a GEMM of `tiles` tiles split into s K parts.  With
// R = tiles / 256 full rounds of the grid and rem tiles left over, splitting
// only the rem tiles takes R s + ceil(rem s / 256) rounds of 1/s tile, exactly
// the ceil(tiles s / 256) rounds of splitting every tile, and writes and
// reduces fp32 partials for the rem tiles only.
int64_t ksplit_t0(int64_t tiles, int s) {
  const int64_t R = tiles / 256, rem = tiles % 256;
  return (s > 1 && R > 0 && rem > 0) ? R * 256 : 0;
}

// fp32 partial floats a split store GEMM needs (0 without a split); `forced`
// is the plan's ksplit (0: the model above).
int64_t kpart_floats(const Ctx& c, int64_t M, int64_t N, int64_t K, int forced = 0) {
  if (!c.bf16) return 0;
  const int s = forced > 0 ? forced : gemm_ksplit(c, M, N, K);
  return s > 1 ? s * M * N : 0;
}

// The plan's value ranges (every call and workspace query; ngemm: GEMMs in
// the call).
lora_status plan_ranges(const Ctx& c, int ngemm) {
  if (c.plan == nullptr || !c.bf16) return LORA_OK;
  for (int i = 0; i < 2; ++i) {
    const lora_gemm_plan& g = c.plan->gemm[i];
    if (i >= ngemm) {
      CHECK(g.group == 0 && g.ksplit == 0, LORA_EINVAL, "plan.gemm[%d] must be zero: the call has %d GEMM", i, ngemm);
      continue;
    }
    const int gr = g.group;
    CHECK(gr == 0 || gr == 1 || gr == 2 || gr == 4 || gr == 8 || gr == 16 || gr == 32, LORA_EINVAL,
          "plan.gemm[%d].group = %d is not 0, 1, 2, 4, 8, 16 or 32", i, gr);
    CHECK(g.ksplit >= 0 && g.ksplit <= 4, LORA_EINVAL, "plan.gemm[%d].ksplit = %d is not in [0, 4]", i, g.ksplit);
  }
  return LORA_OK;
}

// Split-K entry of plan GEMM i of a call (before anything is enqueued):
// splittable = a dense bf16 plain-store GEMM with one output region, of
// [M, N] over K (LoRA tile included).
lora_status plan_split(const Ctx& c, int i, bool splittable, int64_t M, int64_t N, int64_t K) {
  const lora_gemm_plan g = gemm_plan(c, i);
  if (g.ksplit <= 1) return LORA_OK;
  CHECK(splittable, LORA_EINVAL,
        "plan.gemm[%d].ksplit = %d: only a dense plain-store GEMM with one output region can split K", i, g.ksplit);
  CHECK(K / 64 >= g.ksplit, LORA_EINVAL, "plan.gemm[%d].ksplit = %d exceeds the %lld K steps", i, g.ksplit,
        (long long)(K / 64));
  CHECK(M * N * 4 < ((int64_t)1 << 31) - 4096, LORA_EINVAL,
        "plan.gemm[%d]: the fp32 split-K part [%lld, %lld] would exceed 2 GiB", i, (long long)M, (long long)N);
  return LORA_OK;
}

// kpart: fp32 scratch of kpart_floats() for a split store GEMM (nullptr: no
// split); gi: the GEMM's index in the call's plan.
hipError_t gemm_on(const Ctx& c, GemmArgs& g, hipStream_t st, int64_t lora_vcols, int gi, float* kpart = nullptr) {
  const lora_gemm_plan gp = gemm_plan(c, gi);
  g.group = gp.group > 0 ? gp.group : (g.epi == EPI_STORE ? 8 : 4);
  g.lora_vcols = lora_vcols;
  if (c.bf16 && g.RL > 0) {
    // The bf16 kernel runs the LoRA term as one more 64-wide K segment:
    // A = AL [M, 64], B = the packed adapter operand in the main operand's
    // orientation ([64, vcols] for NN, [vcols, 64] for NT), offset to each
    // region's / column group's first virtual column.
    GemmSeg& S = g.seg[g.nseg];
    S = GemmSeg{};
    S.A = g.AL;
    S.lda = g.ldal;
    S.K = g.RL;
    for (int p = 0; p < g.nreg; ++p)
      for (int cg = 0; cg < 2; ++cg) {
        const int64_t v0 = g.reg[p].vcol0[cg];
        BSrc& b = S.b[p][cg];
        if (g.bkind == B_NN) {
          b.p = static_cast<const char*>(g.BLt) + v0 * 2;
          b.ld = lora_vcols;
        } else {
          b.p = static_cast<const char*>(g.BLt) + v0 * g.RL * 2;
          b.ld = g.RL;
        }
      }
    g.nseg += 1;
    g.RL = 0;
  }
  const int64_t rows = gemm_tile_rows(c.bf16);
  const int64_t cols = gemm_tile_cols(c.bf16, g.dual != 0);
  g.ntile_m = cdiv(g.M, rows);
  int64_t tiles = 0;
  for (int p = 0; p < g.nreg; ++p) {
    g.reg[p].tile0 = tiles;
    tiles += cdiv(g.reg[p].N, cols);
  }
  g.ntile_n = tiles;
  g.ksplit = 1;
  if (kpart != nullptr && c.bf16 && !g.nf4 && g.epi == EPI_STORE && g.nreg == 1) {
    int64_t K = 0;
    for (int s = 0; s < g.nseg; ++s) K += g.seg[s].K;
    const int ks = gp.ksplit > 0 ? gp.ksplit : gemm_ksplit(c, g.M, g.reg[0].N, K);
    if (ks > 1) {
      g.ksplit = ks;
      g.ksplit_t0 = (int32_t)ksplit_t0(g.ntile_m * g.ntile_n, ks);
      g.kpart = kpart;
    }
  }
  char name[48];
  std::snprintf(name, sizeof name, "gemm_%s_%s%s%s", g.bkind == B_NN ? "nn" : "nt",
                g.epi == EPI_STORE      ? "store"
                : g.epi == EPI_ACT_FWD  ? "act_fwd"
                : g.epi == EPI_ACT_BWD  ? "act_bwd"
                : g.epi == EPI_ACT1_FWD ? "relu2_fwd"
                                        : "relu2_bwd",
                g.nf4 ? "_nf4" : "", c.bf16 ? "" : "_f32");
  TraceScope ts(name, st);
  if (!c.bf16) return launch_gemm_f32(g, st);
  const hipError_t e = launch_gemm_bf16(g, st);
  if (e != hipSuccess || g.ksplit <= 1) return e;
  return launch_ksplit_reduce(g, st);
}

RowProjArgs rowproj_args(const void* Z, int64_t ldz, int64_t T, int64_t K, const void* Bt, int64_t ldb,
                         int R, int R2, int seg_w) {
  RowProjArgs a{};
  a.Z = Z;
  a.ldz = ldz;
  a.T = T;
  a.K = K;
  a.Bt = Bt;
  a.ldb = ldb;
  a.R = R;
  a.R2 = R2;
  a.seg_w = seg_w;
  return a;
}

// Every colproj output is an adapter gradient: fp32 in the fp32 LoRA-gradient mode.
ColProjArgs colproj_args(const Ctx& c, const void* Z, int64_t ldz, int64_t T, int64_t K, const void* P, int64_t ldp,
                         int R, int seg_w, bool transposed, float* partial) {
  ColProjArgs a{};
  a.out_f32 = c.f32lora ? 1 : 0;
  a.Z = Z;
  a.ldz = ldz;
  a.T = T;
  a.K = K;
  a.P = P;
  a.ldp = ldp;
  a.R = R;
  a.seg_w = seg_w;
  a.transposed = transposed ? 1 : 0;
  a.partial = partial;
  return a;
}

PackPart part(const void* src, int64_t ld, int64_t v0, int64_t nv, int k0, int w, bool nn) {
  PackPart p{};
  p.src = src;
  p.ld = ld;
  p.v0 = v0;
  p.nv = nv;
  p.k0 = k0;
  p.w = w;
  p.nn = nn ? 1 : 0;
  return p;
}

// The adapter-operand packs of one call, issued as one launch before the
// first kernel that reads them.
struct PackBatch {
  PackBatchArgs b{};
  void add(const PackLoraArgs& a) { b.job[b.njobs++] = a; }
  // [A_0 | A_1 | ...]^T, K-contiguous: out [Rpad, K] from A_q [K, w]
  void add_cat_t(void* out, int64_t K, int Rpad, int w, int nparts, const void* const* srcs) {
    PackLoraArgs a{};
    a.out = out;
    a.vcols = K;
    a.RL = Rpad;
    a.nparts = nparts;
    a.kmajor = 1;
    for (int q = 0; q < nparts; ++q) a.part[q] = part(srcs[q], w, 0, K, q * w, w, false);
    add(a);
  }
};

lora_status check_ws(const void* ws, size_t have, size_t need) {
  CHECK(have >= need, LORA_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", have, need);
  CHECK(need == 0 || ws != nullptr, LORA_EWORKSPACE, "workspace is NULL");
  CHECK(aligned(ws, 16), LORA_EALIGN, "workspace is not 16-byte aligned");
  return LORA_OK;
}

// fp32 LoRA-gradient mode: each call first casts its fp32 adapters to bf16
// (round to nearest even) into its workspace and then runs the bf16 path on
// the casts.  The cast area comes first in both workspaces.
struct AdapterDims {
  int64_t n_in, n_out;
};

int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

size_t staged_bytes(const Ctx& c, const AdapterDims* d, int n, int64_t r) {
  if (!c.f32lora) return 0;
  int64_t b = 0;
  for (int i = 0; i < n; ++i) b += round256(d[i].n_in * r * 2) + round256(r * d[i].n_out * 2);
  return (size_t)b;
}

// out[i] = in[i] with A, B replaced by their bf16 casts in `area` (the
// staged_bytes area) when c.f32lora, else a plain copy.  Returns the cast
// launch's arguments (no segments unless c.f32lora).
CastArgs stage_adapters(const Ctx& c, void* area, const lora_proj* const* in, const AdapterDims* d, int n,
                        int64_t r, lora_proj* out) {
  CastArgs a{};
  char* q = static_cast<char*>(area);
  for (int i = 0; i < n; ++i) {
    out[i] = *in[i];
    if (!c.f32lora) continue;
    uint16_t* Ab = reinterpret_cast<uint16_t*>(q);
    q += round256(d[i].n_in * r * 2);
    uint16_t* Bb = reinterpret_cast<uint16_t*>(q);
    q += round256(r * d[i].n_out * 2);
    a.seg[a.nseg++] = CastSeg{static_cast<const float*>(in[i]->A), Ab, d[i].n_in * r};
    a.seg[a.nseg++] = CastSeg{static_cast<const float*>(in[i]->B), Bb, r * d[i].n_out};
    out[i].A = Ab;
    out[i].B = Bb;
  }
  return a;
}

#define STAGE(area, in, dims, n, r, out, st)                      \
  do {                                                            \
    const CastArgs ca_ = stage_adapters(c, area, in, dims, n, r, out); \
    if (c.f32lora) LAUNCHN("cast", st, launch_cast_bf16(ca_, st)); \
  } while (0)

float* partial_buf(Ws& w, const Ctx& c, int64_t T, int64_t K, int R) {
  if (!c.bf16) return nullptr;
  return static_cast<float*>(w.take((size_t)colproj_partial_floats(T, K, R) * 4));
}

// ---------------------------------------------------------------------------
// MLP
// ---------------------------------------------------------------------------
// The bf16 backward GEMM of an MLP forms the down projection's dA in its
// epilogue (rank <= 16): per-m-tile partials of h^T (s P_d), then a
// fixed-order reduce; h itself is never stored in the backward.
bool fuse_da(const Ctx& c, int64_t r) { return c.bf16 && r <= 16; }
int64_t fused_da_floats(int64_t T, int64_t I) { return cdiv(T, gemm_tile_rows(true)) * I * 16; }
// Under the same condition the epilogue also forms the rank-r products of the
// gradients it writes (P = dZ B^T and U^T dZ, per-tile partials): the pass
// over those gradients is replaced by its reduce.

struct MlpPlan {
  void *ad_f, *ad_b;  // adapter casts (fp32 LoRA-gradient mode), fwd / bwd workspace
  void *At_gu, *Us_gu, *BLt_gu, *h, *At_d, *Us_d, *BLt_d;                  // forward
  float* kpart;                                                             // down GEMM split-K
  float* upart;  // h A_d partials of the gate/up epilogue [I/128, T, 16] (fused, bf16, r <= 16)
  void *Ps_d, *BLt_dh, *hb, *dg, *de, *Ps_ug, *BLt_dx;                      // backward
  float* partial;
  float* rpartial;  // rowproj partials of the fused dY pass, then of the batched dg and de passes
  size_t fwd_bytes, bwd_bytes;
};

MlpPlan plan_mlp(const Ctx& c, const lora_mlp_desc& d, void* ws_fwd, void* ws_bwd) {
  MlpPlan p{};
  const int64_t T = d.T, H = d.H, I = d.I, r = d.r;
  const int64_t RLg = c.rl(2 * r), RLd = c.rl(r);
  const AdapterDims ad[3] = {{H, I}, {H, I}, {I, H}};
  Ws f(ws_fwd);
  p.ad_f = f.take(staged_bytes(c, ad, 3, r));
  p.At_gu = f.take(2 * r * H * c.es);
  p.Us_gu = f.take(T * RLg * c.es);
  p.BLt_gu = f.take(2 * I * RLg * c.es);
  p.h = f.take(T * I * c.es);
  p.At_d = f.take(r * I * c.es);
  p.Us_d = f.take(T * RLd * c.es);
  p.BLt_d = f.take(H * RLd * c.es);
  p.kpart = static_cast<float*>(f.take((size_t)kpart_floats(c, T, H, I + RLd, gemm_plan(c, 1).ksplit) * 4));
  p.upart = fuse_da(c, r) ? static_cast<float*>(f.take((size_t)(cdiv(I, gemm_tile_cols(true, true)) * T * 16 * 4)))
                          : nullptr;
  p.fwd_bytes = f.off;
  Ws b(ws_bwd);
  p.ad_b = b.take(staged_bytes(c, ad, 3, r));
  p.Ps_d = b.take(T * RLd * c.es);
  p.BLt_dh = b.take(I * RLd * c.es);
  p.hb = fuse_da(c, r) ? nullptr : b.take(T * I * c.es);
  p.dg = b.take(T * I * c.es);
  p.de = b.take(T * I * c.es);
  p.Ps_ug = b.take(T * RLg * c.es);
  p.BLt_dx = b.take(H * RLg * c.es);
  int64_t pf = 0;
  if (c.bf16) {
    const int64_t cands[4] = {colproj_partial_floats(T, H, (int)r), colproj_partial_floats(T, I, (int)r),
                              colproj_partial_floats(T, H, (int)(2 * r)), 0};
    for (int i = 0; i < 3; ++i) pf = cands[i] > pf ? cands[i] : pf;
    // the dh epilogue's partials: dA_d, then the column products over dg and de
    if (fuse_da(c, r) && 3 * fused_da_floats(T, I) > pf) pf = 3 * fused_da_floats(T, I);
    // the batched dg / de passes (r > 16): one colproj partial per gradient
    const int64_t Kb[2] = {I, I};
    const int64_t bp = 2 * rowcol_batch_partial_floats(T, Kb, 2, 0);
    if (bp > pf) pf = bp;
    // the dX GEMM's split-K partials (the partial buffer is free by then)
    const int64_t kx = kpart_floats(c, T, H, 2 * I + RLg, gemm_plan(c, 1).ksplit);
    if (kx > pf) pf = kx;
  }
  p.partial = static_cast<float*>(b.take((size_t)pf * 4));
  {
    const int64_t rp_dy = rowcol_partial_floats(T, H), rp_gu = 2 * rowcol_partial_floats(T, I);
    p.rpartial = c.bf16 ? static_cast<float*>(b.take((size_t)(rp_dy > rp_gu ? rp_dy : rp_gu) * 4)) : nullptr;
  }
  p.bwd_bytes = b.off;
  return p;
}

lora_status validate_mlp(const lora_mlp_desc* d, Ctx& c) {
  CHECK(d != nullptr, LORA_EINVAL, "desc is NULL");
  TRY(check_dtype(d->dtype, c, true));
  c.plan = d->plan;
  TRY(plan_ranges(c, 2));
  CHECK(d->act == LORA_ACT_SWIGLU || d->act == LORA_ACT_GEGLU_TANH, LORA_EINVAL, "unknown activation %d", d->act);
  CHECK(d->T >= 0, LORA_ESHAPE, "T = %lld is negative", (long long)d->T);
  TRY(check_dim(c, d->H, "H"));
  TRY(check_dim(c, d->I, "I"));
  TRY(check_rank(c, d->r, 2));
  TRY(check_extent(c, d->T, d->I > d->H ? d->I : d->H, "an activation"));
  TRY(check_extent(c, d->H, d->I, "a weight"));
  return LORA_OK;
}


// ---------------------------------------------------------------------------
// Ungated ReLU^2 MLP
// ---------------------------------------------------------------------------
struct Relu2Plan {
  void *ad_f, *ad_b;                                          // adapter casts (fp32 LoRA-gradient mode)
  void *At_u, *Us_u, *BLt_u, *h, *At_d, *Us_d, *BLt_d;        // forward
  float* kpart;                                               // down GEMM split-K
  float* upart;  // h A_d partials of the up GEMM's epilogue [I/256, T, 16] (fused, bf16, r <= 16)
  void *Ps_d, *BLt_dh, *hb, *du, *Ps_u, *BLt_dx;              // backward
  float* partial;
  float* rpartial;  // rowproj partials of the fused dY / du passes
  size_t fwd_bytes, bwd_bytes;
};

Relu2Plan plan_relu2(const Ctx& c, const lora_relu2_mlp_desc& d, void* ws_fwd, void* ws_bwd) {
  Relu2Plan p{};
  const int64_t T = d.T, H = d.H, I = d.I, r = d.r;
  const int64_t RL = c.rl(r);
  const AdapterDims ad[2] = {{H, I}, {I, H}};
  Ws f(ws_fwd);
  p.ad_f = f.take(staged_bytes(c, ad, 2, r));
  p.At_u = f.take(r * H * c.es);
  p.Us_u = f.take(T * RL * c.es);
  p.BLt_u = f.take(I * RL * c.es);
  p.h = f.take(T * I * c.es);
  p.At_d = f.take(r * I * c.es);
  p.Us_d = f.take(T * RL * c.es);
  p.BLt_d = f.take(H * RL * c.es);
  p.kpart = static_cast<float*>(f.take((size_t)kpart_floats(c, T, H, I + RL, gemm_plan(c, 1).ksplit) * 4));
  p.upart = fuse_da(c, r) ? static_cast<float*>(f.take((size_t)(cdiv(I, gemm_tile_cols(true, false)) * T * 16 * 4)))
                          : nullptr;
  p.fwd_bytes = f.off;
  Ws b(ws_bwd);
  p.ad_b = b.take(staged_bytes(c, ad, 2, r));
  p.Ps_d = b.take(T * RL * c.es);
  p.BLt_dh = b.take(I * RL * c.es);
  p.hb = fuse_da(c, r) ? nullptr : b.take(T * I * c.es);
  p.du = b.take(T * I * c.es);
  p.Ps_u = b.take(T * RL * c.es);
  p.BLt_dx = b.take(H * RL * c.es);
  int64_t pf = 0;
  if (c.bf16) {
    const int64_t a = colproj_partial_floats(T, H, (int)r), bb = colproj_partial_floats(T, I, (int)r);
    pf = a > bb ? a : bb;
    // the dh epilogue's partials: dA_d, then the column products over du
    if (fuse_da(c, r) && 2 * fused_da_floats(T, I) > pf) pf = 2 * fused_da_floats(T, I);
    const int64_t kx = kpart_floats(c, T, H, I + RL, gemm_plan(c, 1).ksplit);  // dX split-K
    if (kx > pf) pf = kx;
  }
  p.partial = static_cast<float*>(b.take((size_t)pf * 4));
  p.rpartial = c.bf16 ? static_cast<float*>(b.take((size_t)rowcol_partial_floats(T, I > H ? I : H) * 4)) : nullptr;
  p.bwd_bytes = b.off;
  return p;
}

lora_status validate_relu2(const lora_relu2_mlp_desc* d, Ctx& c) {
  CHECK(d != nullptr, LORA_EINVAL, "desc is NULL");
  TRY(check_dtype(d->dtype, c, true));
  c.plan = d->plan;
  TRY(plan_ranges(c, 2));
  CHECK(d->reserved == 0, LORA_EINVAL, "reserved field must be 0");
  CHECK(d->T >= 0, LORA_ESHAPE, "T = %lld is negative", (long long)d->T);
  TRY(check_dim(c, d->H, "H"));
  TRY(check_dim(c, d->I, "I"));
  TRY(check_rank(c, d->r, 1));
  TRY(check_extent(c, d->T, d->I > d->H ? d->I : d->H, "an activation"));
  TRY(check_extent(c, d->H, d->I, "a weight"));
  return LORA_OK;
}

// ---------------------------------------------------------------------------
// Q/K/V and O
// ---------------------------------------------------------------------------
struct QkvPlan {
  void *ad_f, *ad_b;       // adapter casts (fp32 LoRA-gradient mode)
  void *At, *Us, *BLt;     // forward
  void *Ps, *BLt_dx;       // backward
  float* partial;
  float* rpartial;         // rowproj partials of the batched dQ / dK / dV passes, one region each
  size_t fwd_bytes, bwd_bytes;
};

QkvPlan plan_qkv(const Ctx& c, const lora_qkv_desc& d, void* wf, void* wb) {
  QkvPlan p{};
  const int64_t T = d.T, H = d.H, r = d.r, N = d.Nq + d.Nk + d.Nv;
  const int64_t RL = c.rl(3 * r);
  const AdapterDims ad[3] = {{H, d.Nq}, {H, d.Nk}, {H, d.Nv}};
  Ws f(wf);
  p.ad_f = f.take(staged_bytes(c, ad, 3, r));
  p.At = f.take(3 * r * H * c.es);
  p.Us = f.take(T * RL * c.es);
  p.BLt = f.take(N * RL * c.es);
  p.fwd_bytes = f.off;
  Ws b(wb);
  p.ad_b = b.take(staged_bytes(c, ad, 3, r));
  p.Ps = b.take(T * RL * c.es);
  p.BLt_dx = b.take(H * RL * c.es);
  int64_t pf = 0;
  if (c.bf16) {
    // the batched dQ / dK / dV passes (one colproj partial each), the dA pass over X
    const int64_t Kb[3] = {d.Nq, d.Nk, d.Nv};
    const int64_t cand[2] = {rowcol_batch_partial_floats(T, Kb, 3, 0) + rowcol_batch_partial_floats(T, Kb, 3, 1) +
                                 rowcol_batch_partial_floats(T, Kb, 3, 2),
                             colproj_partial_floats(T, H, (int)(3 * r))};
    for (int i = 0; i < 2; ++i) pf = cand[i] > pf ? cand[i] : pf;
    const int64_t kx = kpart_floats(c, T, H, N + RL, gemm_plan(c, 0).ksplit);  // dX split-K
    if (kx > pf) pf = kx;
  }
  p.partial = static_cast<float*>(b.take((size_t)pf * 4));
  p.rpartial = c.bf16 ? static_cast<float*>(b.take(
                            (size_t)(rowcol_partial_floats(T, d.Nq) + rowcol_partial_floats(T, d.Nk) +
                                     rowcol_partial_floats(T, d.Nv)) * 4))
                      : nullptr;
  p.bwd_bytes = b.off;
  return p;
}

lora_status validate_qkv(const lora_qkv_desc* d, Ctx& c) {
  CHECK(d != nullptr, LORA_EINVAL, "desc is NULL");
  TRY(check_dtype(d->dtype, c, true));
  c.plan = d->plan;
  TRY(plan_ranges(c, 1));
  CHECK(d->reserved == 0, LORA_EINVAL, "reserved field must be 0");
  CHECK(d->T >= 0, LORA_ESHAPE, "T = %lld is negative", (long long)d->T);
  TRY(check_dim(c, d->H, "H"));
  TRY(check_dim(c, d->Nq, "Nq"));
  TRY(check_dim(c, d->Nk, "Nk"));
  TRY(check_dim(c, d->Nv, "Nv"));
  TRY(check_rank(c, d->r, 3));
  // the widest of X, dX and the three outputs / their gradients, and the widest weight
  int64_t nout = d->Nq > d->Nk ? d->Nq : d->Nk;
  nout = nout > d->Nv ? nout : d->Nv;
  TRY(check_extent(c, d->T, d->H > nout ? d->H : nout, "an activation"));
  TRY(check_extent(c, d->H, nout, "a weight"));
  return LORA_OK;
}

struct OPlan {
  void *ad_f, *ad_b;  // adapter casts (fp32 LoRA-gradient mode)
  void *At, *Us, *BLt, *U_tmp;
  float* kpart;  // forward GEMM split-K
  void *Ps, *BLt_dx;
  float* partial;
  float* rpartial;  // rowproj partials of the fused dY pass
  size_t fwd_bytes, bwd_bytes;
};

// Shared by lora_o_* and lora_nf4_gemm: n_in = K, n_out = N.  split = false
// plans the forward without split-K partials (the GEMM then runs unsplit).
OPlan plan_o(const Ctx& c, int64_t T, int64_t K, int64_t N, int64_t r, bool tmp_u, void* wf, void* wb,
             bool split = true) {
  OPlan p{};
  const int64_t RL = c.rl(r);
  const AdapterDims ad[1] = {{K, N}};
  Ws f(wf);
  p.ad_f = f.take(staged_bytes(c, ad, 1, r));
  p.At = f.take(r * K * c.es);
  p.Us = f.take(T * RL * c.es);
  p.BLt = f.take(N * RL * c.es);
  p.U_tmp = tmp_u ? f.take(T * r * c.es) : nullptr;
  p.kpart = split ? static_cast<float*>(f.take((size_t)kpart_floats(c, T, N, K + (r > 0 ? RL : 0), gemm_plan(c, 0).ksplit) * 4)) : nullptr;
  p.fwd_bytes = f.off;
  Ws b(wb);
  p.ad_b = b.take(staged_bytes(c, ad, 1, r));
  p.Ps = b.take(T * RL * c.es);
  p.BLt_dx = b.take(K * RL * c.es);
  int64_t pf = 0;
  if (c.bf16) {
    const int64_t a = colproj_partial_floats(T, N, (int)r), bb = colproj_partial_floats(T, K, (int)r);
    pf = a > bb ? a : bb;
    const int64_t kp = kpart_floats(c, T, K, N + (r > 0 ? RL : 0), gemm_plan(c, 0).ksplit);  // input-gradient split-K
    pf = kp > pf ? kp : pf;
  }
  p.partial = static_cast<float*>(b.take((size_t)pf * 4));
  p.rpartial = c.bf16 ? static_cast<float*>(b.take((size_t)rowcol_partial_floats(T, N) * 4)) : nullptr;
  p.bwd_bytes = b.off;
  return p;
}

lora_status validate_o(const lora_o_desc* d, Ctx& c) {
  CHECK(d != nullptr, LORA_EINVAL, "desc is NULL");
  TRY(check_dtype(d->dtype, c, true));
  c.plan = d->plan;
  TRY(plan_ranges(c, 1));
  CHECK(d->reserved == 0, LORA_EINVAL, "reserved field must be 0");
  CHECK(d->T >= 0, LORA_ESHAPE, "T = %lld is negative", (long long)d->T);
  TRY(check_dim(c, d->K, "K"));
  TRY(check_dim(c, d->N, "N"));
  TRY(check_rank(c, d->r, 1));
  TRY(check_extent(c, d->T, d->K > d->N ? d->K : d->N, "an activation"));
  TRY(check_extent(c, d->K, d->N, "the weight"));
  return LORA_OK;
}

// Forward of one projection: Y = X W + s (X A) B, U = X A (to U if non-NULL).
lora_status proj_forward(const Ctx& c, int64_t T, int64_t K, int64_t N, int64_t r, const void* X,
                         const lora_proj* o, void* Y, void* U, const OPlan& p, hipStream_t st) {
  const int64_t RL = c.rl(r);
  const bool lora = r > 0;
  const bool tw = fwd_t(c, {o});
  GemmArgs g{};
  if (lora) {
    // every adapter operand of the call, packed in one launch
    PackBatch pb;
    const void* srcs[1] = {o->A};
    pb.add_cat_t(p.At, K, (int)r, (int)r, 1, srcs);
    PackLoraArgs pl{};
    pl.out = p.BLt;
    pl.vcols = N;
    pl.RL = (int)RL;
    pl.nparts = 1;
    pl.part[0] = part(o->B, N, 0, N, 0, (int)r, true);
    pl.kmajor = c.bf16 && !tw ? 1 : 0;  // the bf16 NN GEMM reads [RL, vcols], NT [vcols, RL]
    pl.perm8 = pl.kmajor && o->nf4 != nullptr;
    pb.add(pl);
    LAUNCHN("pack", st, launch_pack_batch(c.bf16, pb.b, st));
    RowProjArgs ra = rowproj_args(X, K, T, K, p.At, K, (int)r, (int)RL, (int)r);
    ra.scales[0] = o->scale;
    ra.out1 = U;
    ra.ld1 = r;
    ra.out2 = p.Us;
    ra.ld2 = RL;
    LAUNCHN("rowproj", st, launch_rowproj(c.bf16, ra, st));
    g.AL = p.Us;
    g.ldal = RL;
    g.RL = (int)RL;
    g.BLt = p.BLt;
    g.ldbl = RL;
  }
  g.M = T;
  g.nseg = 1;
  g.nreg = 1;
  g.epi = EPI_STORE;
  g.nf4 = o->nf4 != nullptr;
  g.bkind = tw ? B_NT : B_NN;
  g.seg[0].A = X;
  g.seg[0].lda = K;
  g.seg[0].K = K;
  g.seg[0].b[0][0] = tw ? bsrc_t(o, K) : bsrc(o, N);
  g.reg[0].N = N;
  g.reg[0].out = Y;
  g.reg[0].ldo = N;
  LAUNCH(gemm_on(c, g, st, N, 0, p.kpart));
  return LORA_OK;
}

// Input-gradient GEMM of one projection: dX = dY W^T + (s P) A^T with
// s P = Ps [T, RL] (already formed); A rows feed the LoRA tail.
// The adapter operand of an input-gradient GEMM: A [K, r] as the LoRA tail.
PackBatch input_grad_pack(const Ctx& c, int64_t K, int64_t r, const lora_proj* o, const OPlan& p) {
  PackBatch pb;
  PackLoraArgs pl{};
  pl.out = p.BLt_dx;
  pl.vcols = K;
  pl.RL = (int)c.rl(r);
  pl.nparts = 1;
  pl.part[0] = part(o->A, r, 0, K, 0, (int)r, false);
  pb.add(pl);
  return pb;
}

// packed: input_grad_pack's operand is already in place (an earlier launch ran it)
lora_status proj_input_grad(const Ctx& c, int64_t T, int64_t K, int64_t N, int64_t r, const void* dY,
                            const lora_proj* o, void* dX, const OPlan& p, hipStream_t st, bool packed = false) {
  const int64_t RL = c.rl(r);
  GemmArgs g{};
  if (r > 0) {
    if (!packed) {
      const PackBatch pb = input_grad_pack(c, K, r, o, p);
      LAUNCHN("pack", st, launch_pack_batch(c.bf16, pb.b, st));
    }
    g.AL = p.Ps;
    g.ldal = RL;
    g.RL = (int)RL;
    g.BLt = p.BLt_dx;
    g.ldbl = RL;
  }
  g.M = T;
  g.nseg = 1;
  g.nreg = 1;
  g.epi = EPI_STORE;
  g.nf4 = o->nf4 != nullptr;
  g.bkind = B_NT;
  g.seg[0].A = dY;
  g.seg[0].lda = N;
  g.seg[0].K = N;
  g.seg[0].b[0][0] = bsrc(o, N);
  g.reg[0].N = K;
  g.reg[0].out = dX;
  g.reg[0].ldo = K;
  LAUNCH(gemm_on(c, g, st, K, 0, p.partial));
  return LORA_OK;
}

// ---------------------------------------------------------------------------
// Static scratch of lora_o_fwd_noalloc: one array per device, allocated with
// the code object when the library is loaded on that device and held until
// the process ends.  In host code `scratch` is a host-side stand-in, not a
// device address: every use goes through the address hipGetSymbolAddress
// returns for the current device, looked up once per device at that
// device's first call.  Every call on a device shares its array.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

lora_status static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  CHECK(e == hipSuccess, LORA_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  CHECK(dev >= 0 && dev < kMaxDevices, LORA_EDEVICE, "device %d is beyond the %d the library tracks", dev, kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      CHECK(e == hipSuccess && p != nullptr, LORA_EDEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
            hipGetErrorString(e));
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return LORA_OK;
}

}  // namespace

extern "C" {

int lora_version(void) { return LORA_MI355X_VERSION; }

const char* lora_strerror(lora_status s) {
  // a C caller may pass any integer: read it as one (loading an enum value
  // outside the enumerators is undefined in C++)
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case LORA_OK: return "success";
    case LORA_EINVAL: return "invalid argument";
    case LORA_ESHAPE: return "unsupported shape";
    case LORA_EDTYPE: return "invalid or mismatched dtype";
    case LORA_EALIGN: return "misaligned pointer";
    case LORA_EWORKSPACE: return "workspace missing or too small";
    case LORA_EUNSUPPORTED: return "unsupported combination";
    case LORA_EDEVICE: return "HIP runtime error";
  }
  return "unknown status";
}

const char* lora_last_error(void) { return g_last_error.c_str(); }

void lora_nf4_codebook(float* out) {
  if (out) std::memcpy(out, kNF4Levels, sizeof(kNF4Levels));
}

lora_status lora_mlp_workspace_size(const lora_mlp_desc* d, size_t* fwd, size_t* bwd) {
  Ctx c{};
  TRY(validate_mlp(d, c));
  MlpPlan p = plan_mlp(c, *d, nullptr, nullptr);
  if (fwd) *fwd = p.fwd_bytes;
  if (bwd) *bwd = p.bwd_bytes;
  return LORA_OK;
}

lora_status lora_mlp_fwd(const lora_mlp_desc* d, const void* X, const lora_proj* gate, const lora_proj* up,
                         const lora_proj* down, void* Y, const lora_mlp_saved* saved, void* ws, size_t ws_bytes,
                         void* stream) {
  Ctx c{};
  TRY(validate_mlp(d, c));
  const int64_t T = d->T, H = d->H, I = d->I, r = d->r;
  TRY(check_tptr(c, X, T, "X"));
  TRY(check_tptr(c, Y, T, "Y"));
  CHECK(saved != nullptr, LORA_EINVAL, "saved is NULL");
  TRY(check_tptr(c, saved->e, T, "saved.e"));
  TRY(check_tptr(c, saved->g, T, "saved.g"));
  TRY(check_tptr(c, saved->U, T, "saved.U"));
  TRY(check_proj(c, gate, H, I, "gate"));
  TRY(check_proj(c, up, H, I, "up"));
  TRY(check_proj(c, down, I, H, "down"));
  CHECK((gate->nf4 != nullptr) == (up->nf4 != nullptr), LORA_EUNSUPPORTED, "gate and up must both be NF4 or both dense");
  CHECK(!overlaps(Y, T * H * c.es, X, T * H * c.es), LORA_EUNSUPPORTED, "Y aliases X");
  TRY(plan_split(c, 0, false, 0, 0, 0));
  TRY(plan_split(c, 1, down->nf4 == nullptr, T, H, I + c.rl(r)));
  MlpPlan need = plan_mlp(c, *d, nullptr, nullptr);
  TRY(check_ws(ws, ws_bytes, need.fwd_bytes));
  if (T == 0) return LORA_OK;
  MlpPlan p = plan_mlp(c, *d, ws, nullptr);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t RLg = c.rl(2 * r), RLd = c.rl(r);
  const lora_proj* in[3] = {gate, up, down};
  const AdapterDims ad[3] = {{H, I}, {H, I}, {I, H}};
  lora_proj sp[3];
  STAGE(p.ad_f, in, ad, 3, r, sp, st);
  gate = &sp[0];
  up = &sp[1];
  down = &sp[2];
  const bool t_gu = fwd_t(c, {gate, up}), t_d = fwd_t(c, {down});
  // every adapter operand of the call, packed in one launch
  PackBatch pb;
  const void* srcs_gu[2] = {gate->A, up->A};
  pb.add_cat_t(p.At_gu, H, (int)(2 * r), (int)r, 2, srcs_gu);
  PackLoraArgs pl{};
  pl.out = p.BLt_gu;
  pl.vcols = 2 * I;
  pl.RL = (int)RLg;
  pl.nparts = 2;
  pl.part[0] = part(gate->B, I, 0, I, 0, (int)r, true);
  pl.part[1] = part(up->B, I, I, I, (int)r, (int)r, true);
  pl.kmajor = c.bf16 && !t_gu ? 1 : 0;  // the bf16 NN GEMM reads [RL, vcols], NT [vcols, RL]
  pl.perm8 = pl.kmajor && gate->nf4 != nullptr;
  pb.add(pl);
  const void* srcs_d[1] = {down->A};
  pb.add_cat_t(p.At_d, I, (int)r, (int)r, 1, srcs_d);
  PackLoraArgs pd{};
  pd.out = p.BLt_d;
  pd.vcols = H;
  pd.RL = (int)RLd;
  pd.nparts = 1;
  pd.part[0] = part(down->B, H, 0, H, 0, (int)r, true);
  pd.kmajor = c.bf16 && !t_d ? 1 : 0;
  pd.perm8 = pd.kmajor && down->nf4 != nullptr;
  pb.add(pd);
  LAUNCHN("pack", st, launch_pack_batch(c.bf16, pb.b, st));

  // adapter inputs of gate and up in one pass over X: [U_g | U_u] = X [A_g | A_u]
  RowProjArgs ra = rowproj_args(X, H, T, H, p.At_gu, H, (int)(2 * r), (int)RLg, (int)r);
  ra.scales[0] = gate->scale;
  ra.scales[1] = up->scale;
  ra.out1 = saved->U;
  ra.ld1 = 3 * r;
  ra.off1 = 0;
  ra.out2 = p.Us_gu;
  ra.ld2 = RLg;
  LAUNCHN("rowproj", st, launch_rowproj(c.bf16, ra, st));

  // gate/up GEMM with the activation epilogue
  GemmArgs g{};
  g.M = T;
  g.nseg = 1;
  g.nreg = 1;
  g.dual = 1;
  g.epi = EPI_ACT_FWD;
  g.act = d->act;
  g.nf4 = gate->nf4 != nullptr;
  g.bkind = t_gu ? B_NT : B_NN;
  g.seg[0].A = X;
  g.seg[0].lda = H;
  g.seg[0].K = H;
  g.seg[0].b[0][0] = t_gu ? bsrc_t(gate, H) : bsrc(gate, I);
  g.seg[0].b[0][1] = t_gu ? bsrc_t(up, H) : bsrc(up, I);
  g.reg[0].N = I;
  g.reg[0].vcol0[0] = 0;
  g.reg[0].vcol0[1] = I;
  g.AL = p.Us_gu;
  g.ldal = RLg;
  g.RL = (int)RLg;
  g.BLt = p.BLt_gu;
  g.ldbl = RLg;
  g.e_out = saved->e;
  g.g_out = saved->g;
  g.h_out = p.h;
  g.ld_act = I;
  const bool fu = fuse_da(c, r);  // U_d = h A_d formed in the gate/up epilogue
  if (fu) {
    g.u_part = p.upart;
    g.ad_t = p.At_d;
    g.ld_adt = I;
    g.u_R = (int)r;
  }
  LAUNCH(gemm_on(c, g, st, 2 * I, 0));

  // U_d = h A_d, then the down GEMM
  RowProjArgs rd = rowproj_args(p.h, I, T, I, p.At_d, I, (int)r, (int)RLd, (int)r);
  rd.scales[0] = down->scale;
  rd.out1 = saved->U;
  rd.ld1 = 3 * r;
  rd.off1 = 2 * r;
  rd.out2 = p.Us_d;
  rd.ld2 = RLd;
  if (fu) {
    LAUNCHN("rowproj", st, launch_rowproj_reduce(rd, p.upart, (int)cdiv(I, gemm_tile_cols(true, true)), st));
  } else {
    LAUNCHN("rowproj", st, launch_rowproj(c.bf16, rd, st));
  }

  GemmArgs gd{};
  gd.M = T;
  gd.nseg = 1;
  gd.nreg = 1;
  gd.epi = EPI_STORE;
  gd.nf4 = down->nf4 != nullptr;
  gd.bkind = t_d ? B_NT : B_NN;
  gd.seg[0].A = p.h;
  gd.seg[0].lda = I;
  gd.seg[0].K = I;
  gd.seg[0].b[0][0] = t_d ? bsrc_t(down, I) : bsrc(down, H);
  gd.reg[0].N = H;
  gd.reg[0].out = Y;
  gd.reg[0].ldo = H;
  gd.AL = p.Us_d;
  gd.ldal = RLd;
  gd.RL = (int)RLd;
  gd.BLt = p.BLt_d;
  gd.ldbl = RLd;
  LAUNCH(gemm_on(c, gd, st, H, 1, p.kpart));
  return LORA_OK;
}

lora_status lora_mlp_bwd(const lora_mlp_desc* d, const void* dY, const void* X, const lora_mlp_saved* saved,
                         const lora_proj* gate, const lora_proj* up, const lora_proj* down, void* dX,
                         const lora_mlp_grads* gr, void* ws, size_t ws_bytes, void* stream) {
  Ctx c{};
  TRY(validate_mlp(d, c));
  const int64_t T = d->T, H = d->H, I = d->I, r = d->r;
  TRY(check_tptr(c, dY, T, "dY"));
  TRY(check_tptr(c, X, T, "X"));
  TRY(check_tptr(c, dX, T, "dX"));
  CHECK(saved != nullptr, LORA_EINVAL, "saved is NULL");
  TRY(check_tptr(c, saved->e, T, "saved.e"));
  TRY(check_tptr(c, saved->g, T, "saved.g"));
  TRY(check_tptr(c, saved->U, T, "saved.U"));
  CHECK(gr != nullptr, LORA_EINVAL, "grads is NULL");
  TRY(check_ptr(c, gr->dA_gate, "dA_gate"));
  TRY(check_ptr(c, gr->dB_gate, "dB_gate"));
  TRY(check_ptr(c, gr->dA_up, "dA_up"));
  TRY(check_ptr(c, gr->dB_up, "dB_up"));
  TRY(check_ptr(c, gr->dA_down, "dA_down"));
  TRY(check_ptr(c, gr->dB_down, "dB_down"));
  TRY(check_proj(c, gate, H, I, "gate"));
  TRY(check_proj(c, up, H, I, "up"));
  TRY(check_proj(c, down, I, H, "down"));
  CHECK((gate->nf4 != nullptr) == (up->nf4 != nullptr), LORA_EUNSUPPORTED, "gate and up must both be NF4 or both dense");
  CHECK(dX == X || !overlaps(dX, T * H * c.es, X, T * H * c.es), LORA_EUNSUPPORTED, "dX partly overlaps X");
  TRY(plan_split(c, 0, false, 0, 0, 0));
  TRY(plan_split(c, 1, gate->nf4 == nullptr, T, H, 2 * I + c.rl(2 * r)));
  MlpPlan need = plan_mlp(c, *d, nullptr, nullptr);
  TRY(check_ws(ws, ws_bytes, need.bwd_bytes));
  MlpPlan p = plan_mlp(c, *d, nullptr, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t RLg = c.rl(2 * r), RLd = c.rl(r);
  const lora_proj* in[3] = {gate, up, down};
  const AdapterDims ad[3] = {{H, I}, {H, I}, {I, H}};
  lora_proj sp[3];
  STAGE(p.ad_b, in, ad, 3, r, sp, st);
  gate = &sp[0];
  up = &sp[1];
  down = &sp[2];
  const void* U = saved->U;
  // every adapter operand of the call, packed in one launch (with the reduce below)
  PackBatch pb;
  PackLoraArgs pl{};
  pl.out = p.BLt_dh;
  pl.vcols = I;
  pl.RL = (int)RLd;
  pl.nparts = 1;
  pl.part[0] = part(down->A, r, 0, I, 0, (int)r, false);
  pb.add(pl);
  PackLoraArgs px{};
  px.out = p.BLt_dx;
  px.vcols = H;
  px.RL = (int)RLg;
  px.nparts = 2;
  px.part[0] = part(up->A, r, 0, H, 0, (int)r, false);
  px.part[1] = part(gate->A, r, 0, H, (int)r, (int)r, false);
  pb.add(px);

  // one pass over dY: P_d = dY B_d^T, formed once (scaled copy feeds dA_d and
  // the dh GEMM), and dB_d = s_d U_d^T dY; the launch of its reduce also
  // packs the adapter operands above, which the GEMMs read
  RowProjArgs r1 = rowproj_args(dY, H, T, H, down->B, H, (int)r, (int)RLd, (int)r);
  r1.scales[0] = down->scale;
  r1.out2 = p.Ps_d;
  r1.ld2 = RLd;
  ColProjArgs c1 = colproj_args(c, dY, H, T, H, coff(U, 2 * r, c), 3 * r, (int)r, (int)r, true, p.partial);
  c1.scales[0] = down->scale;
  c1.dest[0] = gr->dB_down;
  LAUNCHN("rowcol", st, launch_rowcol(c.bf16, c1, r1, p.rpartial, st, &pb.b));

  // dh GEMM with the activation-gradient epilogue -> dg, de, h
  GemmArgs g{};
  g.M = T;
  g.nseg = 1;
  g.nreg = 1;
  g.epi = EPI_ACT_BWD;
  g.act = d->act;
  g.nf4 = down->nf4 != nullptr;
  g.bkind = B_NT;
  g.seg[0].A = dY;
  g.seg[0].lda = H;
  g.seg[0].K = H;
  g.seg[0].b[0][0] = bsrc(down, H);
  g.reg[0].N = I;
  g.AL = p.Ps_d;
  g.ldal = RLd;
  g.RL = (int)RLd;
  g.BLt = p.BLt_dh;
  g.ldbl = RLd;
  g.e_in = saved->e;
  g.g_in = saved->g;
  g.dg_out = p.dg;
  g.de_out = p.de;
  g.ld_act = I;
  const bool fda = fuse_da(c, r);
  if (fda) {
    g.dA_part = p.partial;
    g.pd = p.Ps_d;
    g.ldpd = RLd;
    // rank-r products of dg (p = 0: P_u, dB_u) and de (p = 1: P_g, dB_g)
    g.rc_part[0] = p.partial + fused_da_floats(T, I);
    g.rc_part[1] = p.partial + 2 * fused_da_floats(T, I);
    g.rc_rpart[0] = p.rpartial;
    g.rc_rpart[1] = p.rpartial + rowcol_partial_floats(T, I);
    g.rc_b[0] = up->B;
    g.rc_b[1] = gate->B;
    g.rc_ldb = I;
    g.rc_R = (int)r;
    g.rc_u = U;
    g.rc_ldu = 3 * r;
    g.rc_uoff[0] = (int)r;
    g.rc_uoff[1] = 0;
  } else {
    g.h_out = p.hb;
  }
  LAUNCH(gemm_on(c, g, st, I, 0));

  // dA_d = s_d h^T P_d  (P_d already scaled): the reduce of the epilogue's
  // per-m-tile partials (in the launch of the gradients' reduces), or a pass
  // over the stored h
  ColProjArgs c2 = colproj_args(c, p.hb, I, T, I, p.Ps_d, RLd, (int)r, (int)r, false, p.partial);
  c2.scales[0] = 1.0f;
  c2.dest[0] = gr->dA_down;
  if (fda) {
    c2.nchunk = (int)cdiv(T, gemm_tile_rows(true));  // reduced in the launch of the gradients' reduces below
  } else {
    LAUNCHN("colproj", st, launch_colproj(c.bf16, c2, st));
  }

  // one pass over dg: P_u = dg B_u^T (formed once, into [s_u P_u | s_g P_g])
  // and dB_u = s_u U_u^T dg; the same over de for P_g and dB_g
  RowProjArgs r2 = rowproj_args(p.dg, I, T, I, up->B, I, (int)r, (int)r, (int)r);
  r2.scales[0] = up->scale;
  r2.out2 = p.Ps_ug;
  r2.ld2 = RLg;
  // both passes in one launch, each with scratch of its own (a batch that
  // does not fuse, r > 16, runs them one after the other on the same scratch)
  const int64_t Kb[2] = {I, I};
  const bool rc_fused = c.bf16 && r <= 16;
  float* const part_de = p.partial + (rc_fused ? rowcol_batch_partial_floats(T, Kb, 2, 0) : 0);
  ColProjArgs c3 = colproj_args(c, p.dg, I, T, I, coff(U, r, c), 3 * r, (int)r, (int)r, true, p.partial);
  c3.scales[0] = up->scale;
  c3.dest[0] = gr->dB_up;
  c3.rpartial = p.rpartial;
  RowProjArgs r3 = rowproj_args(p.de, I, T, I, gate->B, I, (int)r, (int)(RLg - r), (int)r);
  r3.scales[0] = gate->scale;
  r3.out2 = offw(p.Ps_ug, r, c);
  r3.ld2 = RLg;
  ColProjArgs c4 = colproj_args(c, p.de, I, T, I, U, 3 * r, (int)r, (int)r, true, part_de);
  c4.scales[0] = gate->scale;
  c4.dest[0] = gr->dB_gate;
  c4.rpartial = rc_fused ? p.rpartial + rowcol_partial_floats(T, I) : p.rpartial;
  if (fda) {
    // the dh epilogue wrote the partials: per-m-tile column products, per-n-tile row products
    c3.partial = g.rc_part[0];
    c4.partial = g.rc_part[1];
    c3.nchunk = c4.nchunk = (int)cdiv(T, gemm_tile_rows(true));
    c3.rpartial = g.rc_rpart[0];
    c4.rpartial = g.rc_rpart[1];
  }
  const ColProjArgs cb[2] = {c3, c4};
  const RowProjArgs rb[2] = {r2, r3};
  if (fda) LAUNCHN("rowcol_reduce", st, launch_rowcol_batch_reduce(cb, rb, 2, &c2, 1, st));
  else LAUNCHN("rowcol", st, launch_rowcol_batch(c.bf16, cb, rb, 2, st));

  // [dA_u | dA_g] = X^T [s_u P_u | s_g P_g] in one pass over X
  ColProjArgs c5 = colproj_args(c, X, H, T, H, p.Ps_ug, RLg, (int)(2 * r), (int)r, false, p.partial);
  c5.scales[0] = 1.0f;
  c5.scales[1] = 1.0f;
  c5.dest[0] = gr->dA_up;
  c5.dest[1] = gr->dA_gate;
  LAUNCHN("colproj", st, launch_colproj(c.bf16, c5, st));

  // dX = dg W_u^T + de W_g^T + [s_u P_u | s_g P_g] [A_u | A_g]^T
  GemmArgs gx{};
  gx.M = T;
  gx.nseg = 2;
  gx.nreg = 1;
  gx.epi = EPI_STORE;
  gx.nf4 = up->nf4 != nullptr;
  gx.bkind = B_NT;
  gx.seg[0].A = p.dg;
  gx.seg[0].lda = I;
  gx.seg[0].K = I;
  gx.seg[0].b[0][0] = bsrc(up, I);
  gx.seg[1].A = p.de;
  gx.seg[1].lda = I;
  gx.seg[1].K = I;
  gx.seg[1].b[0][0] = bsrc(gate, I);
  gx.reg[0].N = H;
  gx.reg[0].out = dX;
  gx.reg[0].ldo = H;
  gx.AL = p.Ps_ug;
  gx.ldal = RLg;
  gx.RL = (int)RLg;
  gx.BLt = p.BLt_dx;
  gx.ldbl = RLg;
  if (T > 0) LAUNCH(gemm_on(c, gx, st, H, 1, p.partial));
  return LORA_OK;
}


// ---------------------------------------------------------------------------
// Ungated ReLU^2 MLP
// ---------------------------------------------------------------------------
lora_status lora_relu2_mlp_workspace_size(const lora_relu2_mlp_desc* d, size_t* fwd, size_t* bwd) {
  Ctx c{};
  TRY(validate_relu2(d, c));
  Relu2Plan p = plan_relu2(c, *d, nullptr, nullptr);
  if (fwd) *fwd = p.fwd_bytes;
  if (bwd) *bwd = p.bwd_bytes;
  return LORA_OK;
}

lora_status lora_relu2_mlp_fwd(const lora_relu2_mlp_desc* d, const void* X, const lora_proj* up,
                               const lora_proj* down, void* Y, const lora_relu2_mlp_saved* saved, void* ws,
                               size_t ws_bytes, void* stream) {
  Ctx c{};
  TRY(validate_relu2(d, c));
  const int64_t T = d->T, H = d->H, I = d->I, r = d->r;
  TRY(check_tptr(c, X, T, "X"));
  TRY(check_tptr(c, Y, T, "Y"));
  CHECK(saved != nullptr, LORA_EINVAL, "saved is NULL");
  TRY(check_tptr(c, saved->u, T, "saved.u"));
  TRY(check_tptr(c, saved->U, T, "saved.U"));
  TRY(check_proj(c, up, H, I, "up"));
  TRY(check_proj(c, down, I, H, "down"));
  CHECK(!overlaps(Y, T * H * c.es, X, T * H * c.es), LORA_EUNSUPPORTED, "Y aliases X");
  TRY(plan_split(c, 0, false, 0, 0, 0));
  TRY(plan_split(c, 1, down->nf4 == nullptr, d->T, d->H, d->I + c.rl(d->r)));
  Relu2Plan need = plan_relu2(c, *d, nullptr, nullptr);
  TRY(check_ws(ws, ws_bytes, need.fwd_bytes));
  if (T == 0) return LORA_OK;
  Relu2Plan p = plan_relu2(c, *d, ws, nullptr);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t RL = c.rl(r);
  const lora_proj* in[2] = {up, down};
  const AdapterDims ad[2] = {{H, I}, {I, H}};
  lora_proj sp[2];
  STAGE(p.ad_f, in, ad, 2, r, sp, st);
  up = &sp[0];
  down = &sp[1];
  const bool t_u = fwd_t(c, {up}), t_d = fwd_t(c, {down});
  // every adapter operand of the call, packed in one launch
  PackBatch pb;
  const void* srcs_u[1] = {up->A};
  pb.add_cat_t(p.At_u, H, (int)r, (int)r, 1, srcs_u);
  PackLoraArgs pu{};
  pu.out = p.BLt_u;
  pu.vcols = I;
  pu.RL = (int)RL;
  pu.nparts = 1;
  pu.part[0] = part(up->B, I, 0, I, 0, (int)r, true);
  pu.kmajor = c.bf16 && !t_u ? 1 : 0;  // the bf16 NN GEMM reads [RL, vcols], NT [vcols, RL]
  pu.perm8 = pu.kmajor && up->nf4 != nullptr;
  pb.add(pu);
  const void* srcs_d[1] = {down->A};
  pb.add_cat_t(p.At_d, I, (int)r, (int)r, 1, srcs_d);
  PackLoraArgs pd{};
  pd.out = p.BLt_d;
  pd.vcols = H;
  pd.RL = (int)RL;
  pd.nparts = 1;
  pd.part[0] = part(down->B, H, 0, H, 0, (int)r, true);
  pd.kmajor = c.bf16 && !t_d ? 1 : 0;
  pd.perm8 = pd.kmajor && down->nf4 != nullptr;
  pb.add(pd);
  LAUNCHN("pack", st, launch_pack_batch(c.bf16, pb.b, st));

  // U_u = X A_u, then the up GEMM with the ReLU^2 epilogue (u, h)
  RowProjArgs ru = rowproj_args(X, H, T, H, p.At_u, H, (int)r, (int)RL, (int)r);
  ru.scales[0] = up->scale;
  ru.out1 = saved->U;
  ru.ld1 = 2 * r;
  ru.off1 = 0;
  ru.out2 = p.Us_u;
  ru.ld2 = RL;
  LAUNCHN("rowproj", st, launch_rowproj(c.bf16, ru, st));
  GemmArgs g{};
  g.M = T;
  g.nseg = 1;
  g.nreg = 1;
  g.epi = EPI_ACT1_FWD;
  g.nf4 = up->nf4 != nullptr;
  g.bkind = t_u ? B_NT : B_NN;
  g.seg[0].A = X;
  g.seg[0].lda = H;
  g.seg[0].K = H;
  g.seg[0].b[0][0] = t_u ? bsrc_t(up, H) : bsrc(up, I);
  g.reg[0].N = I;
  g.AL = p.Us_u;
  g.ldal = RL;
  g.RL = (int)RL;
  g.BLt = p.BLt_u;
  g.ldbl = RL;
  g.e_out = saved->u;
  g.h_out = p.h;
  g.ld_act = I;
  const bool fu = fuse_da(c, r);  // U_d = h A_d formed in the up GEMM's epilogue
  if (fu) {
    g.u_part = p.upart;
    g.ad_t = p.At_d;
    g.ld_adt = I;
    g.u_R = (int)r;
  }
  LAUNCH(gemm_on(c, g, st, I, 0));

  // U_d = h A_d, then the down GEMM
  RowProjArgs rd = rowproj_args(p.h, I, T, I, p.At_d, I, (int)r, (int)RL, (int)r);
  rd.scales[0] = down->scale;
  rd.out1 = saved->U;
  rd.ld1 = 2 * r;
  rd.off1 = r;
  rd.out2 = p.Us_d;
  rd.ld2 = RL;
  if (fu) {
    LAUNCHN("rowproj", st, launch_rowproj_reduce(rd, p.upart, (int)cdiv(I, gemm_tile_cols(true, false)), st));
  } else {
    LAUNCHN("rowproj", st, launch_rowproj(c.bf16, rd, st));
  }
  GemmArgs gd{};
  gd.M = T;
  gd.nseg = 1;
  gd.nreg = 1;
  gd.epi = EPI_STORE;
  gd.nf4 = down->nf4 != nullptr;
  gd.bkind = t_d ? B_NT : B_NN;
  gd.seg[0].A = p.h;
  gd.seg[0].lda = I;
  gd.seg[0].K = I;
  gd.seg[0].b[0][0] = t_d ? bsrc_t(down, I) : bsrc(down, H);
  gd.reg[0].N = H;
  gd.reg[0].out = Y;
  gd.reg[0].ldo = H;
  gd.AL = p.Us_d;
  gd.ldal = RL;
  gd.RL = (int)RL;
  gd.BLt = p.BLt_d;
  gd.ldbl = RL;
  LAUNCH(gemm_on(c, gd, st, H, 1, p.kpart));
  return LORA_OK;
}

lora_status lora_relu2_mlp_bwd(const lora_relu2_mlp_desc* d, const void* dY, const void* X,
                               const lora_relu2_mlp_saved* saved, const lora_proj* up, const lora_proj* down,
                               void* dX, const lora_relu2_mlp_grads* gr, void* ws, size_t ws_bytes,
                               void* stream) {
  Ctx c{};
  TRY(validate_relu2(d, c));
  const int64_t T = d->T, H = d->H, I = d->I, r = d->r;
  TRY(check_tptr(c, dY, T, "dY"));
  TRY(check_tptr(c, X, T, "X"));
  TRY(check_tptr(c, dX, T, "dX"));
  CHECK(saved != nullptr, LORA_EINVAL, "saved is NULL");
  TRY(check_tptr(c, saved->u, T, "saved.u"));
  TRY(check_tptr(c, saved->U, T, "saved.U"));
  CHECK(gr != nullptr, LORA_EINVAL, "grads is NULL");
  TRY(check_ptr(c, gr->dA_up, "dA_up"));
  TRY(check_ptr(c, gr->dB_up, "dB_up"));
  TRY(check_ptr(c, gr->dA_down, "dA_down"));
  TRY(check_ptr(c, gr->dB_down, "dB_down"));
  TRY(check_proj(c, up, H, I, "up"));
  TRY(check_proj(c, down, I, H, "down"));
  CHECK(dX == X || !overlaps(dX, T * H * c.es, X, T * H * c.es), LORA_EUNSUPPORTED, "dX partly overlaps X");
  TRY(plan_split(c, 0, false, 0, 0, 0));
  TRY(plan_split(c, 1, up->nf4 == nullptr, d->T, d->H, d->I + c.rl(d->r)));
  Relu2Plan need = plan_relu2(c, *d, nullptr, nullptr);
  TRY(check_ws(ws, ws_bytes, need.bwd_bytes));
  Relu2Plan p = plan_relu2(c, *d, nullptr, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t RL = c.rl(r);
  const lora_proj* in[2] = {up, down};
  const AdapterDims ad[2] = {{H, I}, {I, H}};
  lora_proj sp[2];
  STAGE(p.ad_b, in, ad, 2, r, sp, st);
  up = &sp[0];
  down = &sp[1];
  const void* U = saved->U;
  // every adapter operand of the call, packed in one launch (with the reduce below)
  PackBatch pb;
  PackLoraArgs pl{};
  pl.out = p.BLt_dh;
  pl.vcols = I;
  pl.RL = (int)RL;
  pl.nparts = 1;
  pl.part[0] = part(down->A, r, 0, I, 0, (int)r, false);
  pb.add(pl);
  PackLoraArgs px{};
  px.out = p.BLt_dx;
  px.vcols = H;
  px.RL = (int)RL;
  px.nparts = 1;
  px.part[0] = part(up->A, r, 0, H, 0, (int)r, false);
  pb.add(px);

  // one pass over dY: P_d = dY B_d^T, formed once (scaled copy feeds dA_d and
  // the dh GEMM), and dB_d = s_d U_d^T dY; the launch of its reduce also
  // packs the adapter operands above, which the GEMMs read
  RowProjArgs r1 = rowproj_args(dY, H, T, H, down->B, H, (int)r, (int)RL, (int)r);
  r1.scales[0] = down->scale;
  r1.out2 = p.Ps_d;
  r1.ld2 = RL;
  ColProjArgs c1 = colproj_args(c, dY, H, T, H, coff(U, r, c), 2 * r, (int)r, (int)r, true, p.partial);
  c1.scales[0] = down->scale;
  c1.dest[0] = gr->dB_down;
  LAUNCHN("rowcol", st, launch_rowcol(c.bf16, c1, r1, p.rpartial, st, &pb.b));

  // dh GEMM with the ReLU^2 gradient epilogue -> du, h
  GemmArgs g{};
  g.M = T;
  g.nseg = 1;
  g.nreg = 1;
  g.epi = EPI_ACT1_BWD;
  g.nf4 = down->nf4 != nullptr;
  g.bkind = B_NT;
  g.seg[0].A = dY;
  g.seg[0].lda = H;
  g.seg[0].K = H;
  g.seg[0].b[0][0] = bsrc(down, H);
  g.reg[0].N = I;
  g.AL = p.Ps_d;
  g.ldal = RL;
  g.RL = (int)RL;
  g.BLt = p.BLt_dh;
  g.ldbl = RL;
  g.e_in = saved->u;
  g.dg_out = p.du;
  g.ld_act = I;
  const bool fda = fuse_da(c, r);
  if (fda) {
    g.dA_part = p.partial;
    g.pd = p.Ps_d;
    g.ldpd = RL;
    // rank-r products of du (P_u, dB_u)
    g.rc_part[0] = p.partial + fused_da_floats(T, I);
    g.rc_rpart[0] = p.rpartial;
    g.rc_b[0] = up->B;
    g.rc_ldb = I;
    g.rc_R = (int)r;
    g.rc_u = U;
    g.rc_ldu = 2 * r;
    g.rc_uoff[0] = 0;
  } else {
    g.h_out = p.hb;
  }
  LAUNCH(gemm_on(c, g, st, I, 0));

  // dA_d = s_d h^T P_d  (P_d already scaled): the reduce of the epilogue's
  // per-m-tile partials (in the launch of the gradients' reduces), or a pass
  // over the stored h
  ColProjArgs c2 = colproj_args(c, p.hb, I, T, I, p.Ps_d, RL, (int)r, (int)r, false, p.partial);
  c2.scales[0] = 1.0f;
  c2.dest[0] = gr->dA_down;
  if (fda) {
    c2.nchunk = (int)cdiv(T, gemm_tile_rows(true));  // reduced in the launch of the gradients' reduces below
  } else {
    LAUNCHN("colproj", st, launch_colproj(c.bf16, c2, st));
  }

  // one pass over du: P_u = du B_u^T (formed once) and dB_u = s_u U_u^T du
  RowProjArgs r2 = rowproj_args(p.du, I, T, I, up->B, I, (int)r, (int)RL, (int)r);
  r2.scales[0] = up->scale;
  r2.out2 = p.Ps_u;
  r2.ld2 = RL;
  ColProjArgs c3 = colproj_args(c, p.du, I, T, I, U, 2 * r, (int)r, (int)r, true, p.partial);
  c3.scales[0] = up->scale;
  c3.dest[0] = gr->dB_up;
  if (fda) {
    // the dh epilogue wrote the partials: per-m-tile column products, per-n-tile row products
    c3.partial = g.rc_part[0];
    c3.nchunk = (int)cdiv(T, gemm_tile_rows(true));
    c3.rpartial = g.rc_rpart[0];
    LAUNCHN("rowcol_reduce", st, launch_rowcol_batch_reduce(&c3, &r2, 1, &c2, 1, st));
  } else {
    LAUNCHN("rowcol", st, launch_rowcol(c.bf16, c3, r2, p.rpartial, st));
  }

  // dA_u = X^T (s_u P_u)
  ColProjArgs c4 = colproj_args(c, X, H, T, H, p.Ps_u, RL, (int)r, (int)r, false, p.partial);
  c4.scales[0] = 1.0f;
  c4.dest[0] = gr->dA_up;
  LAUNCHN("colproj", st, launch_colproj(c.bf16, c4, st));

  // dX = du W_u^T + (s_u P_u) A_u^T
  GemmArgs gx{};
  gx.M = T;
  gx.nseg = 1;
  gx.nreg = 1;
  gx.epi = EPI_STORE;
  gx.nf4 = up->nf4 != nullptr;
  gx.bkind = B_NT;
  gx.seg[0].A = p.du;
  gx.seg[0].lda = I;
  gx.seg[0].K = I;
  gx.seg[0].b[0][0] = bsrc(up, I);
  gx.reg[0].N = H;
  gx.reg[0].out = dX;
  gx.reg[0].ldo = H;
  gx.AL = p.Ps_u;
  gx.ldal = RL;
  gx.RL = (int)RL;
  gx.BLt = p.BLt_dx;
  gx.ldbl = RL;
  if (T > 0) LAUNCH(gemm_on(c, gx, st, H, 1, p.partial));
  return LORA_OK;
}

// ---------------------------------------------------------------------------
// Q/K/V
// ---------------------------------------------------------------------------
lora_status lora_qkv_workspace_size(const lora_qkv_desc* d, size_t* fwd, size_t* bwd) {
  Ctx c{};
  TRY(validate_qkv(d, c));
  QkvPlan p = plan_qkv(c, *d, nullptr, nullptr);
  if (fwd) *fwd = p.fwd_bytes;
  if (bwd) *bwd = p.bwd_bytes;
  return LORA_OK;
}

lora_status lora_qkv_fwd(const lora_qkv_desc* d, const void* X, const lora_proj* q, const lora_proj* k,
                         const lora_proj* v, void* Q, void* K, void* V, void* U, void* ws, size_t ws_bytes,
                         void* stream) {
  Ctx c{};
  TRY(validate_qkv(d, c));
  const int64_t T = d->T, H = d->H, r = d->r, Nq = d->Nq, Nk = d->Nk, Nv = d->Nv;
  TRY(check_tptr(c, X, T, "X"));
  TRY(check_tptr(c, Q, T, "Q"));
  TRY(check_tptr(c, K, T, "K"));
  TRY(check_tptr(c, V, T, "V"));
  TRY(check_tptr(c, U, T, "U"));
  TRY(check_proj(c, q, H, Nq, "q"));
  TRY(check_proj(c, k, H, Nk, "k"));
  TRY(check_proj(c, v, H, Nv, "v"));
  CHECK(((q->nf4 != nullptr) == (k->nf4 != nullptr)) && ((k->nf4 != nullptr) == (v->nf4 != nullptr)),
        LORA_EUNSUPPORTED, "q, k, v must all be NF4 or all dense");
  TRY(plan_split(c, 0, false, 0, 0, 0));
  QkvPlan need = plan_qkv(c, *d, nullptr, nullptr);
  TRY(check_ws(ws, ws_bytes, need.fwd_bytes));
  if (T == 0) return LORA_OK;
  QkvPlan p = plan_qkv(c, *d, ws, nullptr);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t RL = c.rl(3 * r);
  const lora_proj* in[3] = {q, k, v};
  const AdapterDims ad[3] = {{H, Nq}, {H, Nk}, {H, Nv}};
  lora_proj sp[3];
  STAGE(p.ad_f, in, ad, 3, r, sp, st);
  q = &sp[0];
  k = &sp[1];
  v = &sp[2];

  const bool tw = fwd_t(c, {q, k, v});
  // every adapter operand of the call, packed in one launch
  PackBatch pb;
  const void* srcs[3] = {q->A, k->A, v->A};
  pb.add_cat_t(p.At, H, (int)(3 * r), (int)r, 3, srcs);
  PackLoraArgs pl{};
  pl.out = p.BLt;
  pl.vcols = Nq + Nk + Nv;
  pl.RL = (int)RL;
  pl.nparts = 3;
  pl.part[0] = part(q->B, Nq, 0, Nq, 0, (int)r, true);
  pl.part[1] = part(k->B, Nk, Nq, Nk, (int)r, (int)r, true);
  pl.part[2] = part(v->B, Nv, Nq + Nk, Nv, (int)(2 * r), (int)r, true);
  pl.kmajor = c.bf16 && !tw ? 1 : 0;  // the bf16 NN GEMM reads [RL, vcols], NT [vcols, RL]
  pl.perm8 = pl.kmajor && q->nf4 != nullptr;
  pb.add(pl);
  LAUNCHN("pack", st, launch_pack_batch(c.bf16, pb.b, st));

  // [U_q | U_k | U_v] = X [A_q | A_k | A_v] in one pass over X
  RowProjArgs ra = rowproj_args(X, H, T, H, p.At, H, (int)(3 * r), (int)RL, (int)r);
  ra.scales[0] = q->scale;
  ra.scales[1] = k->scale;
  ra.scales[2] = v->scale;
  ra.out1 = U;
  ra.ld1 = 3 * r;
  ra.out2 = p.Us;
  ra.ld2 = RL;
  LAUNCHN("rowproj", st, launch_rowproj(c.bf16, ra, st));

  GemmArgs g{};
  g.M = T;
  g.nseg = 1;
  g.nreg = 3;
  g.epi = EPI_STORE;
  g.nf4 = q->nf4 != nullptr;
  g.bkind = tw ? B_NT : B_NN;
  g.seg[0].A = X;
  g.seg[0].lda = H;
  g.seg[0].K = H;
  g.seg[0].b[0][0] = tw ? bsrc_t(q, H) : bsrc(q, Nq);
  g.seg[0].b[1][0] = tw ? bsrc_t(k, H) : bsrc(k, Nk);
  g.seg[0].b[2][0] = tw ? bsrc_t(v, H) : bsrc(v, Nv);
  const int64_t Ns[3] = {Nq, Nk, Nv};
  void* outs[3] = {Q, K, V};
  int64_t v0 = 0;
  for (int i = 0; i < 3; ++i) {
    g.reg[i].N = Ns[i];
    g.reg[i].out = outs[i];
    g.reg[i].ldo = Ns[i];
    g.reg[i].vcol0[0] = v0;
    v0 += Ns[i];
  }
  g.AL = p.Us;
  g.ldal = RL;
  g.RL = (int)RL;
  g.BLt = p.BLt;
  g.ldbl = RL;
  LAUNCH(gemm_on(c, g, st, Nq + Nk + Nv, 0));
  return LORA_OK;
}

lora_status lora_qkv_bwd(const lora_qkv_desc* d, const void* dQ, const void* dK, const void* dV, const void* X,
                         const void* U, const lora_proj* q, const lora_proj* k, const lora_proj* v, void* dX,
                         const lora_qkv_grads* gr, void* ws, size_t ws_bytes, void* stream) {
  Ctx c{};
  TRY(validate_qkv(d, c));
  const int64_t T = d->T, H = d->H, r = d->r, Nq = d->Nq, Nk = d->Nk, Nv = d->Nv;
  TRY(check_tptr(c, dQ, T, "dQ"));
  TRY(check_tptr(c, dK, T, "dK"));
  TRY(check_tptr(c, dV, T, "dV"));
  TRY(check_tptr(c, X, T, "X"));
  TRY(check_tptr(c, U, T, "U"));
  TRY(check_tptr(c, dX, T, "dX"));
  CHECK(gr != nullptr, LORA_EINVAL, "grads is NULL");
  TRY(check_ptr(c, gr->dA_q, "dA_q"));
  TRY(check_ptr(c, gr->dB_q, "dB_q"));
  TRY(check_ptr(c, gr->dA_k, "dA_k"));
  TRY(check_ptr(c, gr->dB_k, "dB_k"));
  TRY(check_ptr(c, gr->dA_v, "dA_v"));
  TRY(check_ptr(c, gr->dB_v, "dB_v"));
  TRY(check_proj(c, q, H, Nq, "q"));
  TRY(check_proj(c, k, H, Nk, "k"));
  TRY(check_proj(c, v, H, Nv, "v"));
  CHECK(((q->nf4 != nullptr) == (k->nf4 != nullptr)) && ((k->nf4 != nullptr) == (v->nf4 != nullptr)),
        LORA_EUNSUPPORTED, "q, k, v must all be NF4 or all dense");
  CHECK(dX == X || !overlaps(dX, T * H * c.es, X, T * H * c.es), LORA_EUNSUPPORTED, "dX partly overlaps X");
  TRY(plan_split(c, 0, q->nf4 == nullptr, T, H, Nq + Nk + Nv + c.rl(3 * r)));
  QkvPlan need = plan_qkv(c, *d, nullptr, nullptr);
  TRY(check_ws(ws, ws_bytes, need.bwd_bytes));
  QkvPlan p = plan_qkv(c, *d, nullptr, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t RL = c.rl(3 * r);
  const lora_proj* in[3] = {q, k, v};
  const AdapterDims ad[3] = {{H, Nq}, {H, Nk}, {H, Nv}};
  lora_proj sp[3];
  STAGE(p.ad_b, in, ad, 3, r, sp, st);
  q = &sp[0];
  k = &sp[1];
  v = &sp[2];
  const lora_proj* projs[3] = {q, k, v};
  const void* dZ[3] = {dQ, dK, dV};
  const int64_t Ns[3] = {Nq, Nk, Nv};
  void* dBs[3] = {gr->dB_q, gr->dB_k, gr->dB_v};

  // one pass over each dZ_p: P_p = dZ_p B_p^T, formed once into
  // [s_q P_q | s_k P_k | s_v P_v], and dB_p = s_p U_p^T dZ_p
  // (the three passes in one launch, each with scratch of its own)
  RowProjArgs rb[3];
  ColProjArgs cb[3];
  float* cpart = p.partial;
  float* rpart = p.rpartial;
  for (int i = 0; i < 3; ++i) {
    const int R2 = (i == 2) ? (int)(RL - 2 * r) : (int)r;
    RowProjArgs ra = rowproj_args(dZ[i], Ns[i], T, Ns[i], projs[i]->B, Ns[i], (int)r, R2, (int)r);
    ra.scales[0] = projs[i]->scale;
    ra.out2 = offw(p.Ps, i * r, c);
    ra.ld2 = RL;
    ColProjArgs ca = colproj_args(c, dZ[i], Ns[i], T, Ns[i], coff(U, i * r, c), 3 * r, (int)r, (int)r, true, cpart);
    ca.scales[0] = projs[i]->scale;
    ca.dest[0] = dBs[i];
    ca.rpartial = rpart;
    rb[i] = ra;
    cb[i] = ca;
    if (c.bf16) {
      cpart += rowcol_batch_partial_floats(T, Ns, 3, i);
      rpart += rowcol_partial_floats(T, Ns[i]);
    }
  }
  // the adapter operand of the dX GEMM, [A_q | A_k | A_v] as its LoRA tail,
  // packed by the launch of the passes' reduces
  PackLoraArgs pl{};
  pl.out = p.BLt_dx;
  pl.vcols = H;
  pl.RL = (int)RL;
  pl.nparts = 3;
  for (int i = 0; i < 3; ++i) pl.part[i] = part(projs[i]->A, r, 0, H, (int)(i * r), (int)r, false);
  PackBatch pb;
  pb.add(pl);
  LAUNCHN("rowcol", st, launch_rowcol_batch(c.bf16, cb, rb, 3, st, &pb.b));
  // [dA_q | dA_k | dA_v] = X^T [s P] in one pass over X
  ColProjArgs cx = colproj_args(c, X, H, T, H, p.Ps, RL, (int)(3 * r), (int)r, false, p.partial);
  cx.scales[0] = cx.scales[1] = cx.scales[2] = 1.0f;
  cx.dest[0] = gr->dA_q;
  cx.dest[1] = gr->dA_k;
  cx.dest[2] = gr->dA_v;
  LAUNCHN("colproj", st, launch_colproj(c.bf16, cx, st));
  // dX = sum_p dZ_p W_p^T + [s P] [A_q | A_k | A_v]^T
  GemmArgs g{};
  g.M = T;
  g.nseg = 3;
  g.nreg = 1;
  g.epi = EPI_STORE;
  g.nf4 = q->nf4 != nullptr;
  g.bkind = B_NT;
  for (int i = 0; i < 3; ++i) {
    g.seg[i].A = dZ[i];
    g.seg[i].lda = Ns[i];
    g.seg[i].K = Ns[i];
    g.seg[i].b[0][0] = bsrc(projs[i], Ns[i]);
  }
  g.reg[0].N = H;
  g.reg[0].out = dX;
  g.reg[0].ldo = H;
  g.AL = p.Ps;
  g.ldal = RL;
  g.RL = (int)RL;
  g.BLt = p.BLt_dx;
  g.ldbl = RL;
  LAUNCH(gemm_on(c, g, st, H, 0, p.partial));
  return LORA_OK;
}

// ---------------------------------------------------------------------------
// O (single projection)
// ---------------------------------------------------------------------------
lora_status lora_o_workspace_size(const lora_o_desc* d, size_t* fwd, size_t* bwd) {
  Ctx c{};
  TRY(validate_o(d, c));
  OPlan p = plan_o(c, d->T, d->K, d->N, d->r, false, nullptr, nullptr);
  if (fwd) *fwd = p.fwd_bytes;
  if (bwd) *bwd = p.bwd_bytes;
  return LORA_OK;
}

lora_status lora_o_fwd(const lora_o_desc* d, const void* X, const lora_proj* o, void* Y, void* U, void* ws,
                       size_t ws_bytes, void* stream) {
  Ctx c{};
  TRY(validate_o(d, c));
  const int64_t T = d->T;
  TRY(check_tptr(c, X, T, "X"));
  TRY(check_tptr(c, Y, T, "Y"));
  TRY(check_tptr(c, U, T, "U"));
  TRY(check_proj(c, o, d->K, d->N, "o"));
  TRY(plan_split(c, 0, o->nf4 == nullptr, d->T, d->N, d->K + c.rl(d->r)));
  OPlan need = plan_o(c, d->T, d->K, d->N, d->r, false, nullptr, nullptr);
  TRY(check_ws(ws, ws_bytes, need.fwd_bytes));
  if (d->T == 0) return LORA_OK;
  OPlan p = plan_o(c, d->T, d->K, d->N, d->r, false, ws, nullptr);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const AdapterDims ad[1] = {{d->K, d->N}};
  lora_proj sp[1];
  STAGE(p.ad_f, &o, ad, 1, d->r, sp, st);
  return proj_forward(c, d->T, d->K, d->N, d->r, X, &sp[0], Y, U, p, st);
}

lora_status lora_o_fwd_noalloc(const lora_o_desc* d, const void* X, const lora_proj* o, void* Y, void* U,
                               void* stream) {
  Ctx c{};
  TRY(validate_o(d, c));
  const int64_t T = d->T;
  TRY(check_tptr(c, X, T, "X"));
  TRY(check_tptr(c, Y, T, "Y"));
  TRY(check_tptr(c, U, T, "U"));
  TRY(check_proj(c, o, d->K, d->N, "o"));
  // the GEMM runs unsplit here: no fp32 split-K partials in the scratch
  TRY(plan_split(c, 0, false, 0, 0, 0));
  OPlan need = plan_o(c, d->T, d->K, d->N, d->r, false, nullptr, nullptr, false);
  CHECK(need.fwd_bytes <= kScratchBytes, LORA_EWORKSPACE,
        "this call needs %zu bytes of scratch; the static scratch holds %zu (fewer tokens per call fit)",
        need.fwd_bytes, kScratchBytes);
  void* ws = nullptr;
  TRY(static_scratch(&ws));
  if (d->T == 0) return LORA_OK;
  OPlan p = plan_o(c, d->T, d->K, d->N, d->r, false, ws, nullptr, false);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const AdapterDims ad[1] = {{d->K, d->N}};
  lora_proj sp[1];
  STAGE(p.ad_f, &o, ad, 1, d->r, sp, st);
  return proj_forward(c, d->T, d->K, d->N, d->r, X, &sp[0], Y, U, p, st);
}

lora_status lora_o_bwd(const lora_o_desc* d, const void* dY, const void* X, const void* U, const lora_proj* o,
                       void* dX, void* dA, void* dB, void* ws, size_t ws_bytes, void* stream) {
  Ctx c{};
  TRY(validate_o(d, c));
  const int64_t T = d->T, K = d->K, N = d->N, r = d->r;
  TRY(check_tptr(c, dY, T, "dY"));
  TRY(check_tptr(c, X, T, "X"));
  TRY(check_tptr(c, U, T, "U"));
  TRY(check_tptr(c, dX, T, "dX"));
  TRY(check_ptr(c, dA, "dA"));
  TRY(check_ptr(c, dB, "dB"));
  TRY(check_proj(c, o, K, N, "o"));
  CHECK(dX == X || !overlaps(dX, T * K * c.es, X, T * K * c.es), LORA_EUNSUPPORTED, "dX partly overlaps X");
  TRY(plan_split(c, 0, o->nf4 == nullptr, T, K, N + c.rl(r)));
  OPlan need = plan_o(c, T, K, N, r, false, nullptr, nullptr);
  TRY(check_ws(ws, ws_bytes, need.bwd_bytes));
  OPlan p = plan_o(c, T, K, N, r, false, nullptr, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t RL = c.rl(r);
  const AdapterDims ad[1] = {{K, N}};
  lora_proj sp[1];
  STAGE(p.ad_b, &o, ad, 1, r, sp, st);
  o = &sp[0];
  // one pass over dY: P = dY B^T, formed once, and dB = s U^T dY
  RowProjArgs ra = rowproj_args(dY, N, T, N, o->B, N, (int)r, (int)RL, (int)r);
  ra.scales[0] = o->scale;
  ra.out2 = p.Ps;
  ra.ld2 = RL;
  ColProjArgs cb = colproj_args(c, dY, N, T, N, U, r, (int)r, (int)r, true, p.partial);
  cb.scales[0] = o->scale;
  cb.dest[0] = dB;
  // the launch of the pass's reduce also packs the input-gradient GEMM's adapter operand
  const PackBatch pb = input_grad_pack(c, K, r, o, p);
  LAUNCHN("rowcol", st, launch_rowcol(c.bf16, cb, ra, p.rpartial, st, r > 0 ? &pb.b : nullptr));
  // dA = X^T (s P)
  ColProjArgs ca = colproj_args(c, X, K, T, K, p.Ps, RL, (int)r, (int)r, false, p.partial);
  ca.scales[0] = 1.0f;
  ca.dest[0] = dA;
  LAUNCHN("colproj", st, launch_colproj(c.bf16, ca, st));
  if (T == 0) return LORA_OK;
  return proj_input_grad(c, T, K, N, r, dY, o, dX, p, st, true);
}

// ---------------------------------------------------------------------------
// NF4
// ---------------------------------------------------------------------------
lora_status lora_nf4_quantize_workspace_size(int64_t rows, int64_t cols, size_t* bytes) {
  CHECK(rows > 0 && cols > 0, LORA_ESHAPE, "NF4 weight must be non-empty");
  CHECK((rows * cols) % NF4_GROUP == 0, LORA_ESHAPE, "NF4 numel %lld not a multiple of %lld",
        (long long)(rows * cols), (long long)NF4_GROUP);
  if (bytes) *bytes = nf4_quantize_ws_bytes(rows * cols);
  return LORA_OK;
}

lora_status lora_nf4_quantize(const void* W, int64_t rows, int64_t cols, int32_t dtype, uint8_t* codes, int8_t* q8,
                              float* s2, float* mu, void* ws, size_t ws_bytes, void* stream) {
  Ctx c{};
  TRY(check_dtype(dtype, c));
  size_t need = 0;
  TRY(lora_nf4_quantize_workspace_size(rows, cols, &need));
  CHECK(W && codes && q8 && s2 && mu, LORA_EINVAL, "NULL argument");
  CHECK(aligned(W, c.es) && aligned(codes, 16) && aligned(s2, 4) && aligned(mu, 4), LORA_EALIGN,
        "W must be element-aligned, codes 16-byte aligned, s2 and mu 4-byte aligned");
  TRY(check_ws(ws, ws_bytes, need));
  LAUNCHN("nf4_quantize", static_cast<hipStream_t>(stream), launch_nf4_quantize(W, rows * cols, c.bf16, codes, q8, s2, mu, ws, static_cast<hipStream_t>(stream)));
  return LORA_OK;
}

lora_status lora_nf4_dequant(const lora_nf4* w, void* out, int32_t dtype, void* stream) {
  Ctx c{};
  TRY(check_dtype(dtype, c));
  CHECK(w != nullptr && out != nullptr, LORA_EINVAL, "NULL argument");
  CHECK(w->rows > 0 && w->cols > 0, LORA_ESHAPE, "NF4 weight must be non-empty");
  TRY(check_nf4(w, w->rows, w->cols, "W"));
  CHECK(aligned(out, 16), LORA_EALIGN, "out must be 16-byte aligned");
  LAUNCHN("nf4_dequant", static_cast<hipStream_t>(stream), launch_nf4_dequant(w->codes, w->q8, w->s2, w->mu, w->rows * w->cols, out, c.bf16,
                            static_cast<hipStream_t>(stream)));
  return LORA_OK;
}

lora_status lora_nf4_unpack_codes(const lora_nf4* w, uint8_t* out, void* stream) {
  CHECK(w != nullptr && out != nullptr, LORA_EINVAL, "NULL argument");
  CHECK(w->rows > 0 && w->cols > 0, LORA_ESHAPE, "NF4 weight must be non-empty");
  TRY(check_nf4(w, w->rows, w->cols, "W"));
  CHECK(aligned(out, 8), LORA_EALIGN, "out must be 8-byte aligned");
  LAUNCHN("nf4_unpack", static_cast<hipStream_t>(stream), launch_nf4_unpack(w->codes, w->rows * w->cols, out, static_cast<hipStream_t>(stream)));
  return LORA_OK;
}

lora_status lora_nf4_gemm_workspace_size(int64_t T, int64_t rows, int64_t cols, int64_t r, int32_t trans,
                                         size_t* bytes) {
  Ctx c{};
  TRY(check_dtype(LORA_BF16, c));
  CHECK(T >= 0, LORA_ESHAPE, "T is negative");
  CHECK(trans == 0 || trans == 1, LORA_EINVAL, "trans must be 0 or 1");
  TRY(check_dim(c, rows, "rows"));
  TRY(check_dim(c, cols, "cols"));
  if (r != 0) TRY(check_rank(c, r, 1));
  // 32-bit operand offsets: the activations [T, rows | cols] and the weight
  // (its dequantized bf16 extent bounds every NF4 array and element index)
  TRY(check_extent(c, T, rows > cols ? rows : cols, "an activation"));
  TRY(check_extent(c, rows, cols, "the weight"));
  OPlan p = plan_o(c, T, rows, cols, r, trans == 0, nullptr, nullptr);
  if (bytes) *bytes = trans ? p.bwd_bytes : p.fwd_bytes;
  return LORA_OK;
}

lora_status lora_nf4_gemm(int64_t T, int32_t trans, const void* X, const lora_nf4* W, const void* A, const void* B,
                          int64_t r, float scale, void* Y, void* ws, size_t ws_bytes, void* stream) {
  Ctx c{};
  TRY(check_dtype(LORA_BF16, c));
  CHECK(W != nullptr, LORA_EINVAL, "W is NULL");
  CHECK((A == nullptr) == (B == nullptr), LORA_EINVAL, "A and B must both be set or both be NULL");
  const int64_t rr = A ? r : 0;
  size_t need = 0;
  TRY(lora_nf4_gemm_workspace_size(T, W->rows, W->cols, rr, trans, &need));
  TRY(check_tptr(c, X, T, "X"));
  TRY(check_tptr(c, Y, T, "Y"));
  TRY(check_nf4(W, W->rows, W->cols, "W"));
  if (rr > 0) {
    TRY(check_ptr(c, A, "A"));
    TRY(check_ptr(c, B, "B"));
    CHECK(std::isfinite(scale), LORA_EINVAL, "scale is not finite");
  }
  lora_proj o{};
  o.nf4 = W;
  o.A = A;
  o.B = B;
  o.scale = scale;
  TRY(check_ws(ws, ws_bytes, need));
  if (T == 0) return LORA_OK;
  const int64_t K = W->rows, N = W->cols;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (trans == 0) {
    OPlan p = plan_o(c, T, K, N, rr, true, ws, nullptr);
    return proj_forward(c, T, K, N, rr, X, &o, Y, p.U_tmp, p, st);
  }
  OPlan p = plan_o(c, T, K, N, rr, false, nullptr, ws);
  if (rr > 0) {
    const int64_t RL = c.rl(rr);
    RowProjArgs ra = rowproj_args(X, N, T, N, B, N, (int)rr, (int)RL, (int)rr);
    ra.scales[0] = scale;
    ra.out2 = p.Ps;
    ra.ld2 = RL;
    LAUNCHN("rowproj", st, launch_rowproj(c.bf16, ra, st));
  }
  return proj_input_grad(c, T, K, N, rr, X, &o, Y, p, st);
}

}  // extern "C"
