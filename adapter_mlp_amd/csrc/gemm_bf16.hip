// bf16 GEMM core for gfx950: 256x256x64 block tiles, 4 wavefronts (2 x 2),
// each wavefront a 128x128 sub-tile of v_mfma_f32_32x32x16_bf16 products with
// fp32 accumulation, operands staged through double-buffered LDS.
//
// What it computes (the base projections and the adapter term of the LoRA
// projections, "LoRA Optimizations" section "Custom autograd functions"; the
// products of the unsloth LoRA_MLP / LoRA_QKV / LoRA_W hunks):
//   forward   Z = X W + (s X A) B        (B operand [K, N], N-contiguous: "NN")
//   backward  dX = dZ W^T + (s P) A^T    (B operand [N, K], K-contiguous: "NT")
// The adapter term is one more K tile of the same MFMA loop: [X | sU] [W ; B].
//
// Epilogues run on the accumulators right after the K loop:
//   EPI_STORE    round to bf16, store;
//   EPI_ACT_FWD  (gate/up tiles) e, g -> bf16, h = phi(e) g from the rounded
//                e, g, store e, g, h;
//   EPI_ACT_BWD  dh -> load e, g, recompute h, dg = dh phi(e),
//                de = dh g phi'(e), store dg, de, h.
// Each wavefront stages its results through a private LDS region so global
// loads and stores move whole 16-byte chunks of consecutive columns.
//
// MFMA roles.  The weight tile is the MFMA "A" source (32 rows = output
// columns n) and the activation tile the "B" source (32 columns = rows m), so
// each lane ends with 4 consecutive output columns of one row, and the gated
// activation finds e and g of the same element in the same lane.
//
// Operands are read with buffer loads: the descriptor base advances by one K
// tile per step (scalar work only) and rows past the end of a matrix read as
// zero, which covers ragged M and N tiles without clamping.
//
// NN weight tiles (forward) are transposed on the way into LDS: each thread
// loads an 8x8 bf16 sub-block (8 rows of 16 bytes) and transposes it in
// registers with v_perm_b32 before writing 8 K-contiguous 16-byte rows.
//
// NF4 weights are unpacked in registers on the same path: a 32-bit load
// holds 8 codes of one 64-element block; the block's absmax is rebuilt from
// its int8 code, its scaler block's fp32 scale and the global mean, each code
// looks up its level, and fl32(level * absmax) is rounded to bf16 before the
// 16 bytes go to LDS ("loralei" README, section "Use": unpack and
// double-scale reconstruction fused into the matmul).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace lora {
namespace {

constexpr int BM = 256, BK = 64, NTH = 256;
constexpr int TILE_CHUNKS = 256 * 8;  // 16-byte chunks per 256 x 64 bf16 tile
constexpr int OOB = 0x7ffffff0;       // a buffer offset past every operand: loads return 0

// XOR swizzle of the 16-byte chunk index inside a 128-byte LDS row.  Rows read
// together by an MFMA fragment load (8 consecutive rows) and rows written
// together by the transposing store land in different banks.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Buffer descriptor over [p, p + bytes) (bytes < 2^31); every input is uniform.
__device__ __forceinline__ rsrc_t rsrc(const void* p, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  const int64_t base = uni64(reinterpret_cast<int64_t>(p));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ int bload1s(rsrc_t r, int off) {
  return (int)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// Wavefront-local LDS hand-off between lanes (each wavefront stages into its
// own LDS region in the epilogue, so no block barrier is needed).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Block -> tile.  Workgroups are dispatched round-robin over the 8 XCDs, so
// block b runs on XCD b % 8.  Re-number blocks so that each XCD receives a
// contiguous run of logical tiles, and walk logical tiles in groups of 8
// m-tiles (n-major inside a group) so the 32 tiles an XCD holds at once share
// 8 activation panels and 4 weight panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int nb, int ntm, int ntn, int& tm, int& tn) {
  const int q = nb >> 3, rem = nb & 7, x = bid & 7, j = bid >> 3;
  const int lid = (x < rem) ? x * (q + 1) + j : rem * (q + 1) + (x - rem) * q + j;
  const int G = 8;
  const int per_group = G * ntn;
  const int grp = lid / per_group;
  const int first_m = grp * G;
  const int gsize = (ntm - first_m < G) ? (ntm - first_m) : G;
  const int in_g = lid - grp * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

// Tile-local weight row nl (0..255) -> output column.  Dual tiles hold
// [gate 64 | up 64] for wavefront column 0, then the same for column 1.
template <bool DUAL>
__device__ __forceinline__ int64_t colmap(int nl, int64_t tnl) {
  if constexpr (DUAL) return tnl * 128 + (int64_t)(nl >> 7) * 64 + (nl & 63);
  else return tnl * 256 + nl;
}

// 8x8 bf16 transpose: r[i] holds row i (8 values, 2 per dword); o[j] receives
// column j (the 8 row values, 2 per dword).
__device__ __forceinline__ void transpose8x8(const u32x4 (&r)[8], u32x4 (&o)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = r[2 * q][p], hi = r[2 * q + 1][p];
      o[2 * p][q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      o[2 * p + 1][q] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
    }
  }
}

// 8 NF4 codes (one dword, element 2q in the high nibble of byte q) -> 8 bf16.
__device__ __forceinline__ u32x4 nf4_decode8(uint32_t w, float absmax, const float* lut) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t byte = (w >> (8 * q)) & 0xffu;
    const float v0 = __fmul_rn(lut[byte >> 4], absmax);
    const float v1 = __fmul_rn(lut[byte & 0xfu], absmax);
    o[q] = pack_bf2(v0, v1);
  }
  return o;
}

// Calls f(integral_constant<int, 0..3>) so accumulator indices stay
// compile-time constants (a runtime index would move the accumulators to
// scratch memory).
template <typename F>
__device__ __forceinline__ void for4(F&& f) {
  f(std::integral_constant<int, 0>{});
  f(std::integral_constant<int, 1>{});
  f(std::integral_constant<int, 2>{});
  f(std::integral_constant<int, 3>{});
}

struct Stage {
  u32x4 a[8];
  u32x4 b[8];   // dense rows, or b[i][0] = NF4 code dword
  float bs2[8];
  int bq8[8];
};

// Epilogue: each wavefront stages its results (WN output tile columns x 128
// rows; accumulator block i covers tile columns 32 i.., block j rows 32 j..)
// through a private LDS region -- the operand buffers are free once the K
// loop has ended -- so global loads and stores move 16-byte chunks of
// consecutive columns.  In dual tiles blocks i < NI/2 hold gate columns and
// blocks i + NI/2 the up columns of the same outputs.
// Staging bytes one wavefront needs for a WN-column epilogue.
template <int WN, int EPI>
constexpr int epi_stage_bytes() {
  return EPI == EPI_STORE ? 32 * (WN + 8) * 2 : EPI == EPI_ACT_FWD ? 3 * 32 * (WN / 2 + 8) * 2 : 32 * (WN + 4) * 4;
}

template <int WN, bool DUAL, int EPI>
__device__ __forceinline__ void run_epilogue_w(f32x16 (&acc)[WN / 32][4], char* wstage, const GemmArgs& args,
                                               int reg, int64_t mw, int64_t nbase, int64_t NR, int64_t M,
                                               int lane) {
  constexpr int NI = WN / 32;
  if constexpr (EPI == EPI_STORE) {
    constexpr int LD = WN + 8;           // bf16 staging [32][WN], padded rows
    constexpr int CPR = WN / 8;          // 16-byte chunks per row
    constexpr int RPP = 64 / CPR;        // rows per pass
    uint16_t* stg = reinterpret_cast<uint16_t*>(wstage);
    char* out = static_cast<char*>(args.reg[reg].out);
    const int64_t ldo = args.reg[reg].ldo;
    for4([&](auto jc) {
      constexpr int j = decltype(jc)::value;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = i * 32 + 8 * g + 4 * (lane >> 5);
          u32x2 v;
          v[0] = pack_bf2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
          v[1] = pack_bf2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *reinterpret_cast<u32x2*>(stg + (lane & 31) * LD + col) = v;
        }
      wave_sync();
#pragma unroll
      for (int it = 0; it < 32 / RPP; ++it) {
        const int row = it * RPP + lane / CPR, c8 = lane % CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * LD + c8 * 8);
        const int64_t m = mw + j * 32 + row;
        const int64_t n = nbase + c8 * 8;
        if (m < M && n < NR) *reinterpret_cast<u32x4*>(out + (m * ldo + n) * 2) = v;
      }
      wave_sync();
    });
  } else if constexpr (EPI == EPI_ACT_FWD) {
    static_assert(DUAL, "activation forward needs gate/up tiles");
    constexpr int W2 = WN / 2;           // output columns per wavefront
    constexpr int LD = W2 + 8;
    constexpr int ARR = 32 * LD;
    constexpr int CPR = W2 / 8;
    constexpr int RPP = 64 / CPR;
    uint16_t* stg = reinterpret_cast<uint16_t*>(wstage);
    char* eo = static_cast<char*>(args.e_out);
    char* go = static_cast<char*>(args.g_out);
    char* ho = static_cast<char*>(args.h_out);
    const int64_t ld = args.ld_act;
    for4([&](auto jc) {
      constexpr int j = decltype(jc)::value;
#pragma unroll
      for (int i = 0; i < NI / 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = i * 32 + 8 * g + 4 * (lane >> 5);
          u32x2 ev, gv, hv;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            ev[h] = pack_bf2(acc[i][j][4 * g + 2 * h], acc[i][j][4 * g + 2 * h + 1]);
            gv[h] = pack_bf2(acc[i + NI / 2][j][4 * g + 2 * h], acc[i + NI / 2][j][4 * g + 2 * h + 1]);
            float p0, p1;
            act_fwd<false>(args.act, lo_bf(ev[h]), p0);
            act_fwd<false>(args.act, hi_bf(ev[h]), p1);
            hv[h] = pack_bf2(p0 * lo_bf(gv[h]), p1 * hi_bf(gv[h]));
          }
          const int o = (lane & 31) * LD + col;
          *reinterpret_cast<u32x2*>(stg + o) = ev;
          *reinterpret_cast<u32x2*>(stg + ARR + o) = gv;
          *reinterpret_cast<u32x2*>(stg + 2 * ARR + o) = hv;
        }
      wave_sync();
#pragma unroll
      for (int it = 0; it < 32 / RPP; ++it) {
        const int row = it * RPP + lane / CPR, c8 = lane % CPR;
        const int64_t m = mw + j * 32 + row;
        const int64_t n = nbase + c8 * 8;
        if (m < M && n < NR) {
          const int o = row * LD + c8 * 8;
          const int64_t off = (m * ld + n) * 2;
          *reinterpret_cast<u32x4*>(eo + off) = *reinterpret_cast<const u32x4*>(stg + o);
          *reinterpret_cast<u32x4*>(go + off) = *reinterpret_cast<const u32x4*>(stg + ARR + o);
          *reinterpret_cast<u32x4*>(ho + off) = *reinterpret_cast<const u32x4*>(stg + 2 * ARR + o);
        }
      }
      wave_sync();
    });
  } else {
    constexpr int LD = WN + 4;           // fp32 staging [32][WN]
    constexpr int CPR = WN / 8;          // 8-float groups per row
    constexpr int RPP = 64 / CPR;
    constexpr int PASSES = 32 / RPP;
    float* stg = reinterpret_cast<float*>(wstage);
    const char* ei = static_cast<const char*>(args.e_in);
    const char* gi = static_cast<const char*>(args.g_in);
    char* dgo = static_cast<char*>(args.dg_out);
    char* deo = static_cast<char*>(args.de_out);
    char* ho = static_cast<char*>(args.h_out);
    const int64_t ld = args.ld_act;
    for4([&](auto jc) {
      constexpr int j = decltype(jc)::value;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = i * 32 + 8 * g + 4 * (lane >> 5);
          *reinterpret_cast<f32x4*>(stg + (lane & 31) * LD + col) =
              f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
      wave_sync();
      u32x4 ev[PASSES], gv[PASSES];
      f32x4 d0[PASSES], d1[PASSES];
#pragma unroll
      for (int it = 0; it < PASSES; ++it) {
        const int row = it * RPP + lane / CPR, c8 = lane % CPR;
        const int64_t m = mw + j * 32 + row;
        const int64_t n = nbase + c8 * 8;
        const bool ok = m < M && n < NR;
        const int64_t off = ok ? (m * ld + n) * 2 : 0;
        ev[it] = ok ? *reinterpret_cast<const u32x4*>(ei + off) : u32x4{0, 0, 0, 0};
        gv[it] = ok ? *reinterpret_cast<const u32x4*>(gi + off) : u32x4{0, 0, 0, 0};
        d0[it] = *reinterpret_cast<const f32x4*>(stg + row * LD + c8 * 8);
        d1[it] = *reinterpret_cast<const f32x4*>(stg + row * LD + c8 * 8 + 4);
      }
#pragma unroll
      for (int it = 0; it < PASSES; ++it) {
        const int row = it * RPP + lane / CPR, c8 = lane % CPR;
        const int64_t m = mw + j * 32 + row;
        const int64_t n = nbase + c8 * 8;
        u32x4 dgv, dev, hv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float dha = q < 2 ? d0[it][2 * q] : d1[it][2 * q - 4];
          const float dhb = q < 2 ? d0[it][2 * q + 1] : d1[it][2 * q - 3];
          const float e0 = lo_bf(ev[it][q]), e1 = hi_bf(ev[it][q]);
          const float g0 = lo_bf(gv[it][q]), g1 = hi_bf(gv[it][q]);
          float p0, s0, p1, s1;
          act_fwd_bwd<false>(args.act, e0, p0, s0);
          act_fwd_bwd<false>(args.act, e1, p1, s1);
          hv[q] = pack_bf2(p0 * g0, p1 * g1);
          dgv[q] = pack_bf2(dha * p0, dhb * p1);
          dev[q] = pack_bf2(dha * g0 * s0, dhb * g1 * s1);
        }
        if (m < M && n < NR) {
          const int64_t off = (m * ld + n) * 2;
          *reinterpret_cast<u32x4*>(dgo + off) = dgv;
          *reinterpret_cast<u32x4*>(deo + off) = dev;
          *reinterpret_cast<u32x4*>(ho + off) = hv;
        }
      }
      wave_sync();
    });
  }
}

template <bool DUAL, int EPI>
__device__ __forceinline__ void run_epilogue(f32x16 (&acc)[4][4], u32x4* smem, const GemmArgs& args, int reg,
                                             int64_t m0, int64_t tnl, int64_t NR, int64_t M, int wave, int lane) {
  const int wm = wave >> 1, wn = wave & 1;
  char* wstage = reinterpret_cast<char*>(smem) + wave * epi_stage_bytes<128, EPI>();
  run_epilogue_w<128, DUAL, EPI>(acc, wstage, args, reg, m0 + wm * 128, colmap<DUAL>(wn * 128, tnl), NR, M, lane);
}

// NF4 weights: the previous loop (register prefetch of one tile, LoRA tile
// through its own path), kept while the dense kernel is tuned.
template <int BKIND, bool NF4, bool DUAL, int EPI>
__global__ __launch_bounds__(NTH, 1) void gemm_nf4_kernel(const GemmArgs args) {
  __shared__ u32x4 smem[4 * TILE_CHUNKS];  // A: 2 buffers, B: 2 buffers; reused by the epilogue
  __shared__ float s_lut[16];
  u32x4* const sA = smem;
  u32x4* const sB = smem + 2 * TILE_CHUNKS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  if (NF4 && tid < 16) {
    const float lv[16] = LORA_NF4_LEVELS_INIT;
    s_lut[tid] = lv[tid];
  }

  // Tile coordinates are uniform; keep them (and all that derives from them)
  // in scalar registers so buffer descriptors stay scalar.
  int tm, tn;
  tile_coords((int)blockIdx.x, (int)gridDim.x, (int)args.ntile_m, (int)args.ntile_n, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  int reg = 0;
#pragma unroll
  for (int p = 1; p < 3; ++p)
    if (p < args.nreg && tn >= args.reg[p].tile0) reg = p;
  reg = __builtin_amdgcn_readfirstlane(reg);
  const int64_t tnl = uni64(tn - args.reg[reg].tile0);
  const int64_t NR = uni64(args.reg[reg].N);
  const int64_t M = args.M;
  const int64_t m0 = (int64_t)tm * BM;

  // Per-thread load geometry.
  //  A and NT weights: 16-byte chunk a_c of rows a_r0 + 32 i.
  //  NN weights: wavefront w owns tile columns 64w..64w+63 (one column group
  //  of a dual tile); lane = 8 k8 + n8 loads K rows 8 k8..+7, columns 8 n8..+7.
  const int a_c = tid & 7;
  const int a_r0 = tid >> 3;
  const int nn_n8 = lane & 7, nn_k8 = lane >> 3;
  const int nn_cg = DUAL ? (wave & 1) : 0;
  const int64_t nn_col = colmap<DUAL>(wave * 64 + nn_n8 * 8, tnl);

  int64_t ktiles = 0;
  for (int s = 0; s < args.nseg; ++s) ktiles += args.seg[s].K / BK;
  const bool has_lora = args.RL > 0;
  const int64_t KT = ktiles + (has_lora ? 1 : 0);

  // Segment state (uniform): current segment and the K offset inside it.
  int seg = 0;
  int64_t k0 = 0;
  int a_off[8];  // byte offsets of this thread's 8 A rows (OOB past M)
  int b_off[8];  // dense: byte offsets of its 8 weight rows; NF4: element index
  auto seg_setup = [&](int s) {
    const GemmSeg& S = args.seg[s];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + a_r0 + 32 * i;
      a_off[i] = m < M ? (int)((m * S.lda + a_c * 8) * 2) : OOB;
    }
    if constexpr (BKIND == B_NT) {
      const BSrc& B = S.b[reg][0];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t n = colmap<DUAL>(a_r0 + 32 * i, tnl);
        if constexpr (NF4) b_off[i] = n < NR ? (int)(n * B.wcols + a_c * 8) : OOB;
        else b_off[i] = n < NR ? (int)((n * B.ld + a_c * 8) * 2) : OOB;
      }
    } else {
      const BSrc& B = S.b[reg][nn_cg];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (NF4) b_off[i] = (int)((nn_k8 * 8 + i) * B.wcols + nn_col);
        else b_off[i] = (int)(((nn_k8 * 8 + i) * B.ld + nn_col) * 2);
      }
    }
  };

  // --- global -> registers for one main K tile ---------------------------------
  auto load_main = [&](Stage& st) {
    const GemmSeg& S = args.seg[seg];
    const rsrc_t ra = rsrc(static_cast<const char*>(S.A) + k0 * 2, M * S.lda * 2 - k0 * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.a[i] = bload16(ra, a_off[i]);
    const BSrc& B = S.b[reg][BKIND == B_NN ? nn_cg : 0];
    if constexpr (NF4) {
      // weight rows x cols = (NT: N x K_s, NN: K_s x N); tile start in elements
      const int64_t numel = (BKIND == B_NT ? NR : S.K) * B.wcols;
      const int64_t kofs = BKIND == B_NT ? k0 : k0 * B.wcols;
      const rsrc_t rc = rsrc(B.codes + kofs / 2, numel / 2 - kofs / 2);
      const rsrc_t rq = rsrc(B.q8, numel / 64);
      const rsrc_t rs = rsrc(B.s2, (numel / NF4_GROUP) * 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = b_off[i] != OOB;
        const uint32_t flat = (uint32_t)b_off[i] + (uint32_t)kofs;
        st.b[i][0] = bload4(rc, ok ? (int)((uint32_t)b_off[i] >> 1) : OOB);
        st.bq8[i] = bload1s(rq, ok ? (int)(flat >> 6) : OOB);
        st.bs2[i] = __uint_as_float(bload4(rs, ok ? (int)((flat >> 14) << 2) : OOB));
      }
    } else {
      const int64_t total = BKIND == B_NT ? NR * B.ld * 2 : ((S.K - 1) * B.ld + NR) * 2;
      const int64_t adv = (BKIND == B_NT ? k0 : k0 * B.ld) * 2;
      const rsrc_t rb = rsrc(static_cast<const char*>(B.p) + adv, total - adv);
#pragma unroll
      for (int i = 0; i < 8; ++i) st.b[i] = bload16(rb, b_off[i]);
    }
  };

  // NF4 codes -> bf16 (at LDS-store time, after the loads have landed).
  auto decode_nf4 = [&](Stage& st) {
    if constexpr (NF4) {
      const float mu = *args.seg[seg].b[reg][BKIND == B_NN ? nn_cg : 0].mu;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        st.b[i] = nf4_decode8(st.b[i][0], nf4_absmax((int8_t)st.bq8[i], st.bs2[i], mu), s_lut);
    } else {
      (void)st;
    }
  };

  // --- the LoRA tile: A_L [M, RL] and BLt [vcols, RL], both K-contiguous -----
  auto load_lora = [&](Stage& st) {
    const rsrc_t ra = rsrc(args.AL, M * args.ldal * 2);
    const rsrc_t rb = rsrc(args.BLt, args.lora_vcols * args.ldbl * 2);
    const bool chunk_ok = a_c < (args.RL >> 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + a_r0 + 32 * i;
      st.a[i] = bload16(ra, (chunk_ok && m < M) ? (int)((m * args.ldal + a_c * 8) * 2) : OOB);
      const int64_t n = colmap<DUAL>(a_r0 + 32 * i, tnl);
      const int64_t v = args.reg[reg].vcol0[DUAL ? ((i >> 1) & 1) : 0] + n;
      st.b[i] = bload16(rb, (chunk_ok && n < NR) ? (int)((v * args.ldbl + a_c * 8) * 2) : OOB);
    }
  };

  // --- registers -> LDS ---------------------------------------------------------
  auto store_tile = [&](const Stage& st, int buf, bool kcontig_b) {
    u32x4* dA = sA + buf * TILE_CHUNKS;
    u32x4* dB = sB + buf * TILE_CHUNKS;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = a_r0 + 32 * i;
      dA[row * 8 + (a_c ^ swz(row))] = st.a[i];
    }
    if (kcontig_b) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = a_r0 + 32 * i;
        dB[row * 8 + (a_c ^ swz(row))] = st.b[i];
      }
    } else {
      u32x4 cols[8];
      transpose8x8(st.b, cols);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = wave * 64 + nn_n8 * 8 + j;
        dB[row * 8 + (nn_k8 ^ swz(row))] = cols[j];
      }
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // 4 K-steps of 16 over one LDS buffer; fragments of step s+1 are read while
  // the MFMAs of step s issue.
  auto compute = [&](int buf) {
    const u32x4* tA = sA + buf * TILE_CHUNKS;
    const u32x4* tB = sB + buf * TILE_CHUNKS;
    bf16x8 fa[2][4], fb[2][4];
    auto frags = [&](int ks, bf16x8 (&xa)[4], bf16x8 (&xb)[4]) {
      const int c = ks * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rn = wn * 128 + i * 32 + (lane & 31);
        xa[i] = __builtin_bit_cast(bf16x8, tB[rn * 8 + (c ^ swz(rn))]);
        const int rm = wm * 128 + i * 32 + (lane & 31);
        xb[i] = __builtin_bit_cast(bf16x8, tA[rm * 8 + (c ^ swz(rm))]);
      }
    };
    frags(0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) frags(ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][i], fb[ks & 1][j], acc[i][j], 0, 0, 0);
    }
  };

  auto advance = [&]() {
    k0 += BK;
    if (k0 >= args.seg[seg].K && seg + 1 < args.nseg) {
      ++seg;
      k0 = 0;
      seg_setup(seg);
    }
  };

  // --- main loop: prefetch tile t+1 into registers while tile t computes ---
  Stage st;
  seg_setup(0);
  load_main(st);
  __syncthreads();  // s_lut ready
  decode_nf4(st);
  store_tile(st, 0, BKIND == B_NT);
  __syncthreads();

  for (int64_t t = 0; t < KT; ++t) {
    const int buf = (int)(t & 1);
    const bool has_next = t + 1 < KT;
    const bool next_lora = has_lora && t + 1 == ktiles;
    if (has_next) {
      if (next_lora) {
        load_lora(st);
      } else {
        advance();
        load_main(st);
      }
    }
    compute(buf);
    if (has_next) {
      if (!next_lora) decode_nf4(st);
      store_tile(st, buf ^ 1, next_lora || BKIND == B_NT);
    }
    __syncthreads();
  }

  run_epilogue<DUAL, EPI>(acc, smem, args, reg, m0, tnl, NR, M, wave, lane);
}


// ---------------------------------------------------------------------------
// Dense weights.  8 wavefronts in two groups of 4, one wavefront of each
// group on every SIMD, working in alternating phases separated by barriers:
// while group 0 runs a cluster of 32 MFMAs on fragments already in its
// registers, group 1 reads the fragments of its next cluster from LDS, and
// then the roles swap -- the SIMD's matrix unit always has one wavefront
// feeding it and LDS latency never sits between two MFMAs.  Each wavefront
// owns a 128x64 sub-tile (8 accumulators of 32x32); group g covers tile rows
// 128 g .. 128 g + 127.
//
// Operands go from global memory straight into LDS (buffer_load_dwordx4 ...
// lds: lane i of a load writes bytes 16 i .. 16 i + 15 of a 1 KB LDS block
// whose base is in M0), two K steps ahead.  The loads are split between the
// groups so that each phase moves the same 32 KB per CU: group 0 loads the
// activation tiles (in its read phase Y) into a 2-slot ring, group 1 the
// weight tiles (in its read phase X) into a 3-slot ring; with three weight
// slots the weights of step t+2 can be written while both groups still read
// those of steps t and t+1.  LDS: 2 x 32 KB + 3 x 32 KB = 160 KB.
//   activation tile: 256 rows x 64 K, 128-byte rows, 16-byte chunk c of row r
//                    stored at c ^ swz(r); read with ds_read_b128;
//   weights, NT:     the same layout over 256 output columns;
//   weights, NN:     two halves of [64 K][128 N] (256-byte rows; for gate/up
//                    tiles half 0 holds gate and half 1 up columns), chunk c
//                    of row k stored at c ^ 4 (k & 3); fragments are read
//                    with ds_read_b64_tr_b16, which hands lane 16 g + i the
//                    4 values of column i that lanes 16 g + 4 j + i / 4 point
//                    at (j = 0..3), i.e. the K-contiguous MFMA operand.
// ---------------------------------------------------------------------------
constexpr int NTH8 = 512;
constexpr int SLOT_BYTES = 32768;
constexpr int A_SLOTS = 2, W_SLOTS = 3;
constexpr int W_RING = A_SLOTS * SLOT_BYTES;  // weight ring after the activation ring
constexpr int LDS_BYTES = (A_SLOTS + W_SLOTS) * SLOT_BYTES;
constexpr int HALF_BYTES = 16384;

template <int BKIND, bool DUAL, int EPI>
__global__ __launch_bounds__(NTH8, 1) void gemm_dense_kernel(const GemmArgs args) {
  static_assert(!(DUAL && BKIND == B_NT), "gate/up tiles read forward (NN) weights");
  __shared__ __attribute__((aligned(1024))) char smem_raw[LDS_BYTES];
  lds_char* const lds = (lds_char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int wm = wave >> 2, wn = wave & 3;                    // wm: the group

  int tm, tn;
  tile_coords((int)blockIdx.x, (int)gridDim.x, (int)args.ntile_m, (int)args.ntile_n, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  int reg = 0;
#pragma unroll
  for (int p = 1; p < 3; ++p)
    if (p < args.nreg && tn >= args.reg[p].tile0) reg = p;
  reg = __builtin_amdgcn_readfirstlane(reg);
  const int64_t tnl = uni64(tn - args.reg[reg].tile0);
  const int64_t NR = uni64(args.reg[reg].N);
  const int64_t M = args.M;
  const int64_t m0 = (int64_t)tm * BM;

  int KT = 0;
  for (int s = 0; s < args.nseg; ++s) KT += (int)(args.seg[s].K / BK);

  // ---- loads: 8 blocks of 1 KB per wavefront and step ----
  // K-contiguous block q = 8 wn + i holds rows 8 q + lane / 8; its row r has
  // swz(r) = (lane / 8) ^ i, so lane takes logical chunk (lane % 8) ^ (lane / 8) ^ i.
  // NN block q' = 8 (wn & 1) + i of half wn >> 1 holds K rows 4 q' + lane / 16,
  // lane takes logical chunk (lane % 16) ^ 4 (lane / 16).
  const int kc_row = wn * 64 + (lane >> 3);
  const int kc_x = (lane & 7) ^ (lane >> 3);
  const int nn_row = (wn & 1) * 32 + (lane >> 4);
  const int nn_chunk = (lane & 15) ^ (4 * ((lane >> 4) & 3));
  // each group walks the K steps with its own cursor (segment, offset)
  int lseg = 0;
  int64_t lk0 = 0;
  auto advance = [&](const GemmSeg& S) {
    lk0 += BK;
    if (lk0 >= S.K) {
      ++lseg;
      lk0 = 0;
    }
  };
  auto issue_a = [&](int slot) {  // group 0: activation tile of the next step
    const GemmSeg& S = args.seg[lseg];
    const uint32_t dst = lds_addr(lds) + slot * SLOT_BYTES + wn * 8 * 1024;
    // opaque copies: keep the per-lane terms from being expanded per block
    // and hoisted out of the K loop (8 live offsets would not fit)
    int x = kc_x, r = kc_row;
    asm volatile("" : "+v"(x), "+v"(r));
    const uint32_t lda2 = (uint32_t)(S.lda * 2);
    const i32x4 ra = rsrc_words(static_cast<const char*>(S.A) + (m0 * S.lda + lk0) * 2,
                                (M - m0) * S.lda * 2 - lk0 * 2);
    const uint32_t base = (uint32_t)r * lda2;
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(ra, base + (uint32_t)((x ^ i) << 4), dst + i * 1024, (uint32_t)(8 * i) * lda2);
    advance(S);
  };
  auto issue_w = [&](int slot) {  // group 1: weight tile of the next step
    const GemmSeg& S = args.seg[lseg];
    const uint32_t wslot = lds_addr(lds) + W_RING + slot * SLOT_BYTES;
    if constexpr (BKIND == B_NT) {
      const BSrc& B = S.b[reg][0];
      int x = kc_x, r = kc_row;
      asm volatile("" : "+v"(x), "+v"(r));
      const uint32_t ld2 = (uint32_t)(B.ld * 2);
      const i32x4 rb = rsrc_words(static_cast<const char*>(B.p) + (tnl * 256 * B.ld + lk0) * 2,
                                  (NR - tnl * 256) * B.ld * 2 - lk0 * 2);
      const uint32_t base = (uint32_t)r * ld2;
      const uint32_t dst = wslot + wn * 8 * 1024;
#pragma unroll
      for (int i = 0; i < 8; ++i) dma16(rb, base + (uint32_t)((x ^ i) << 4), dst + i * 1024, (uint32_t)(8 * i) * ld2);
    } else {
      const int half = wn >> 1;
      const BSrc& B = S.b[reg][DUAL ? half : 0];
      const uint32_t ld2 = (uint32_t)(B.ld * 2);
      const int64_t ncol0 = DUAL ? tnl * 128 : tnl * 256 + half * 128;
      const i32x4 rb = rsrc_words(static_cast<const char*>(B.p) + (lk0 * B.ld + ncol0) * 2,
                                  ((S.K - 1 - lk0) * B.ld + NR - ncol0) * 2);
      int nr = nn_row, nc = nn_chunk;
      asm volatile("" : "+v"(nr), "+v"(nc));
      const uint32_t base = (uint32_t)nr * ld2 + (uint32_t)(nc << 4);
      const uint32_t dst = wslot + half * HALF_BYTES + (wn & 1) * 8 * 1024;
#pragma unroll
      for (int i = 0; i < 8; ++i) dma16(rb, base, dst + i * 1024, (uint32_t)(4 * i) * ld2);
    }
    advance(S);
  };

  // ---- fragment reads ----
  // NN weights: lane s of read h (0, 1) of K slice ks points at K row
  //   16 ks + 8 (g >> 1) + 4 h + (s & 15) / 4 and columns nb + 16 (g & 1) + 4 (s & 3), g = s / 16
  int fa_nn[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int half = DUAL ? i : (wn >> 1);
    const int nb = DUAL ? wn * 32 : (wn & 1) * 64 + 32 * i;
    const int g = lane >> 4;
    const int n = nb + 16 * (g & 1) + 4 * (lane & 3);
    const int kr = (lane & 15) >> 2;  // K row & 3 of every read of this lane
    fa_nn[i] = half * HALF_BYTES + (8 * (g >> 1) + kr) * 256 + (((n >> 3) ^ (4 * kr)) * 16) + (lane & 1) * 8;
  }
  // K-contiguous tiles: row r0 + 32 j (r0 = first row of the sub-tile + lane % 32)
  // has swz = swz(r0) ^ 4 (j & 1), so chunk 2 ks + lane / 32 sits at
  // (2 ks ^ 4 (j & 1)) ^ x with x = (lane / 32) ^ swz(r0): four per-lane offsets
  // cover every (ks, j); the row term is an immediate.
  auto kc_offsets = [&](int r0, int (&o)[4]) {
    const int x = (lane >> 5) ^ swz(r0);
#pragma unroll
    for (int y = 0; y < 4; ++y) o[y] = r0 * 128 + (((2 * y) ^ x) * 16);
  };
  int ao[4];
  kc_offsets(wm * 128 + (lane & 31), ao);
  int bo[4];
  if constexpr (BKIND == B_NT) kc_offsets(wn * 64 + (lane & 31), bo);

  bf16x8 fa[4][2], fb[4][4];
  auto read = [&](int aslot, int wslot) {
    const lds_char* const at = lds + aslot * SLOT_BYTES;
    const lds_char* const wt = lds + W_RING + wslot * SLOT_BYTES;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (BKIND == B_NN) {
          fa[ks][i] = lds_read_tr8(wt + fa_nn[i] + (16 * ks) * 256, 4 * 256);
        } else {
          const int y = ((2 * ks) ^ (4 * (i & 1))) >> 1;
          fa[ks][i] = __builtin_bit_cast(bf16x8, lds_read16(wt + bo[y] + i * 32 * 128));
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int y = ((2 * ks) ^ (4 * (j & 1))) >> 1;
        fb[ks][j] = __builtin_bit_cast(bf16x8, lds_read16(at + ao[y] + j * 32 * 128));
      }
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  // the MFMA phase runs at raised wavefront priority, so the SIMD's other
  // wavefront (in its read phase) cannot delay the MFMA issue
  auto mma = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- phases.  Every wavefront passes 2 + 2 KT barriers. ----
  //   prologue  g0 loads A 0, 1   g1 loads W 0, 1; each waits for step 0 | barrier
  //             g0 reads step 0                                         | barrier
  //   step t    X: g0 MFMA t, waits for A t+1
  //                g1 loads W t+2, reads step t, waits for W t+1        | barrier
  //             Y: g0 loads A t+2, reads step t+1
  //                g1 MFMA t                                            | barrier
  // A t+2 goes to activation slot t & 1 after its last read (g1, X(t));
  // W t+2 goes to weight slot (t+2) % 3, last read in X(t-1).
  auto phase_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  if (wm == 0) {
    issue_a(0);
    if (KT > 1) {
      issue_a(1);
      __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): A 0 is in
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    phase_end();
    read(0, 0);
    phase_end();
    for (int t = 0; t < KT; ++t) {
      mma();
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): A t+1 is in
      phase_end();
      if (t + 2 < KT) issue_a(t & 1);
      if (t + 1 < KT) read((t + 1) & 1, (t + 1) % 3);
      phase_end();
    }
  } else {
    issue_w(0);
    if (KT > 1) {
      issue_w(1);
      __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): W 0 is in
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    phase_end();
    phase_end();
    int ws = 0;  // weight slot of step t
    for (int t = 0; t < KT; ++t) {
      const int ws2 = ws == 0 ? 2 : ws - 1;  // (t + 2) % 3
      if (t + 2 < KT) {
        issue_w(ws2);
        read(t & 1, ws);
        __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): W t+1 is in (W t+2 may still fly)
      } else {
        read(t & 1, ws);
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      phase_end();
      mma();
      phase_end();
      ws = ws == 2 ? 0 : ws + 1;
    }
  }

  // epilogue staging: a private region per wavefront (operand slots are no longer read)
  constexpr int EB = epi_stage_bytes<64, EPI>();
  static_assert(8 * EB <= LDS_BYTES, "epilogue staging exceeds LDS");
  char* const wstage = smem_raw + wave * EB;
  const int64_t mw = m0 + wm * 128;
  const int64_t nbase = DUAL ? tnl * 128 + wn * 32 : tnl * 256 + wn * 64;
  run_epilogue_w<64, DUAL, EPI>(acc, wstage, args, reg, mw, nbase, NR, M, lane);
}

template <int BKIND, bool DUAL, int EPI>
hipError_t launch_dense(const GemmArgs& a, hipStream_t st) {
  const int64_t nb = a.ntile_m * a.ntile_n;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_dense_kernel<BKIND, DUAL, EPI>), dim3((unsigned)nb), dim3(NTH8), 0, st, a);
  return hipGetLastError();
}

template <int BKIND, bool NF4, bool DUAL, int EPI>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  const int64_t nb = a.ntile_m * a.ntile_n;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_nf4_kernel<BKIND, NF4, DUAL, EPI>), dim3((unsigned)nb), dim3(NTH), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int64_t gemm_tile_cols(bool bf16, bool dual) {
  if (bf16) return dual ? 128 : 256;
  return dual ? 32 : 64;
}
int64_t gemm_tile_rows(bool bf16) { return bf16 ? 256 : 64; }

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t st) {
  if (a.nf4) {
    if (a.bkind == B_NN)
      return a.epi == EPI_ACT_FWD ? launch_t<B_NN, true, true, EPI_ACT_FWD>(a, st)
                                  : launch_t<B_NN, true, false, EPI_STORE>(a, st);
    return a.epi == EPI_ACT_BWD ? launch_t<B_NT, true, false, EPI_ACT_BWD>(a, st)
                                : launch_t<B_NT, true, false, EPI_STORE>(a, st);
  }
  if (a.bkind == B_NN)
    return a.epi == EPI_ACT_FWD ? launch_dense<B_NN, true, EPI_ACT_FWD>(a, st)
                                : launch_dense<B_NN, false, EPI_STORE>(a, st);
  return a.epi == EPI_ACT_BWD ? launch_dense<B_NT, false, EPI_ACT_BWD>(a, st)
                              : launch_dense<B_NT, false, EPI_STORE>(a, st);
}

}  // namespace lora
