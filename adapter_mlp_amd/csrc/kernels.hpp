// Kernel argument structs and host-side launchers shared by the kernel
// translation units and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

// ---------------------------------------------------------------------------
// Tiled GEMM with a LoRA tail and fused epilogues.
//
//   C[m, n] = sum_s sum_k A_s[m, k] B_s[k, n]  +  sum_k AL[m, k] BL[k, n]
//
// Main segments s (at most 3) are concatenated along K; each has its own A
// ([M, K_s] row-major) and, per output region and column group, its own B.
// B orientation is the same for all main segments:
//   B_NN: B_s is [K_s, N] row-major (the weight W [in, out] of a forward);
//   B_NT: B_s is [N, K_s] row-major (W used transposed, an input gradient).
// The LoRA tail AL [M, RL] / BLt [vcols, RL] always comes K-contiguous; BLt
// row v is the adapter column that feeds output column n of region p and
// column group c, v = vcol0[p][c] + n (built by the packing jobs below).
// Up to 3 output regions split the N range (Q/K/V); in "dual" mode every
// tile interleaves two column groups (gate, up) over the same output columns
// so the activation epilogue sees e and g of one element in one lane.
// ---------------------------------------------------------------------------
enum { B_NN = 0, B_NT = 1 };
enum { EPI_STORE = 0, EPI_ACT_FWD = 1, EPI_ACT_BWD = 2, EPI_ACT1_FWD = 3, EPI_ACT1_BWD = 4 };

struct BSrc {
  const void* p;  // dense base (compute dtype) or nullptr for NF4
  int64_t ld;
  const uint8_t* codes;  // NF4
  const int8_t* q8;
  const float* s2;
  const float* mu;
  int64_t wcols;  // row length of the logical NF4 weight
};

struct GemmSeg {
  const void* A;
  int64_t lda;
  int64_t K;
  BSrc b[3][2];  // [region][column group]
};

struct GemmRegion {
  int64_t N;
  int64_t tile0;  // first n-tile of this region
  void* out;      // EPI_STORE output
  int64_t ldo;
  int64_t vcol0[2];
};

struct GemmArgs {
  int64_t M;
  int32_t nseg, nreg;
  int32_t dual, epi, act, nf4, bkind;
  int32_t group;  // m-tiles per group of the XCD-aware tile order (bf16)
  GemmSeg seg[4];  // up to 3 main segments + the LoRA tail as a segment
  GemmRegion reg[3];
  int64_t ntile_m, ntile_n;
  const void* AL;  // LoRA tail (nullptr / RL == 0: none)
  int64_t ldal;
  int32_t RL, pad2_;
  const void* BLt;
  int64_t ldbl;
  int64_t lora_vcols;  // rows of BLt
  // EPI_ACT_FWD: e_out, g_out, h_out [M, N] ; EPI_ACT_BWD: e_in, g_in -> dg_out, de_out, h_out
  // EPI_ACT1_FWD (ungated ReLU^2): e_out = u, h_out ; EPI_ACT1_BWD: e_in = u -> dg_out = du, h_out
  void* e_out;
  void* g_out;
  void* h_out;
  const void* e_in;
  const void* g_in;
  void* dg_out;
  void* de_out;
  int64_t ld_act;
  // bf16 backward epilogues (EPI_ACT_BWD, EPI_ACT1_BWD) with dA_part set: h is
  // not stored; instead each block adds its rows of h^T Pd (Pd [M, ldpd],
  // columns 0..15, the scaled P of the next projection, zero past its rank)
  // into dA_part [ntile_m, N, 16] (fp32, one slice per m-tile), which a
  // fixed-order reduce over the m-tiles turns into dA.
  float* dA_part;
  const void* pd;
  int64_t ldpd;
  // EPI_STORE, bf16, dense, one region: split-K.  Tiles 0 .. ksplit_t0-1 (in
  // the tile order) are computed whole and stored as bf16; each later tile is
  // split into ksplit K parts (the K steps split evenly, in order), block
  // ksplit_t0 + u working on part u / ns of tile ksplit_t0 + u % ns (ns = the
  // split tiles) and writing its fp32 sums to kpart [ksplit, M, N];
  // launch_ksplit_reduce adds the parts of the split tiles in ascending order
  // and stores bf16.  ksplit <= 1: no split.
  int32_t ksplit, ksplit_t0;
  float* kpart;
  // EPI_ACT_FWD (bf16) with u_part set: each block also forms h Ad over its
  // h columns (ad_t = Ad^T [u_R, N], row pitch ld_adt, u_R <= 16) and writes
  // the tile's sums to u_part [ntile_n, M, 16] (fp32); the rowproj reduce
  // adds the n-tile slices in ascending order.
  float* u_part;
  const void* ad_t;
  int64_t ld_adt;
  int32_t u_R, pad4_;
  // bf16 backward epilogues with rc_part[0] set (rank rc_R <= 16): the rank-r
  // products of the gradients the epilogue writes, dZ_0 = dg_out and (gated)
  // dZ_1 = de_out, formed from their bf16 values:
  //   column products U_p^T dZ_p into rc_part[p] [ntile_m, N, 16] (U_p =
  //     columns rc_uoff[p] .. + 15 of rc_u [M, rc_ldu]; sums past the rank
  //     are never read);
  //   row products dZ_p B_p^T into rc_rpart[p] [ntile_n, M, 16] (B_p = rc_b[p]
  //     [rc_R, N], row pitch rc_ldb; zero past the rank);
  // fp32, unscaled, one slice per m-tile or n-tile, which the rowcol reduce
  // adds in a fixed order.
  float* rc_part[2];
  float* rc_rpart[2];
  const void* rc_b[2];
  int64_t rc_ldb;
  const void* rc_u;
  int64_t rc_ldu;
  int32_t rc_uoff[2];
  int32_t rc_R, pad5_;
};

// Columns of output covered by one n-tile.
int64_t gemm_tile_cols(bool bf16, bool dual);
int64_t gemm_tile_rows(bool bf16);
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t st);
// For the split tiles of a (tiles ksplit_t0 ..): out[m, n] (bf16) = sum over
// k < ksplit, ascending, of kpart[k][m][n]
hipError_t launch_ksplit_reduce(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------
// Rank-r products.
// rowproj:  Out[t, j] = sum_k Z[t, k] Bt[j, k]   (j < R, R <= 64)
//   writes out1[t, off1 + j] = Out (unscaled)              if out1
//          out2[t, j] = scale(j) * Out, zero for R <= j < R2   if out2
//   scale(j) = scales[j / seg_w] (seg_w = width of each adapter in the group)
// colproj:  Out[k, j] = sum_t Z[t, k] P[t, j] (j < R)
//   written to dest[q] for j in [q*seg_w, (q+1)*seg_w) times scales[q],
//   transposed ([seg_w, K]) or not ([K, seg_w]).
// ---------------------------------------------------------------------------
struct RowProjArgs {
  const void* Z;
  int64_t ldz, T, K;
  const void* Bt;
  int64_t ldb;
  int32_t R, R2, seg_w, pad_;
  float scales[4];
  void* out1;
  int64_t ld1, off1;
  void* out2;
  int64_t ld2;
};

struct ColProjArgs {
  const void* Z;
  int64_t ldz, T, K;
  const void* P;
  int64_t ldp;
  int32_t R, seg_w, transposed, nchunk;
  float scales[4];
  void* dest[4];
  float* partial;  // bf16 path: [nchunk, K, R] fp32 scratch
  // fused rowproj over the same Z (launch_rowcol): Bt [R1, K] (R1 <= 16),
  // per-column-block partials [K / 256, T, 16] fp32
  const void* Bt;
  int64_t ldb;
  int32_t R1;
  int32_t out_f32;  // bf16 path: dest[] are fp32 (else bf16)
  float* rpartial;
};

hipError_t launch_rowproj(bool bf16, const RowProjArgs& a, hipStream_t st);
hipError_t launch_colproj(bool bf16, const ColProjArgs& a, hipStream_t st);
// Only the reduce of colproj: dest = scales * sum over a.nchunk slices of
// a.partial [nchunk, K, 16] (R <= 16), in ascending slice order.
hipError_t launch_colproj_reduce(const ColProjArgs& a, hipStream_t st);
// rowproj r and colproj c over the same Z [T, K] in one pass (bf16, r.R <= 16):
// the colproj blocks also form r's product over their 256 columns; a
// fixed-order reduce then writes r's outputs.  Other cases run the two
// kernels one after the other.  rpartial: rowcol_partial_floats(T, K) floats.
// With pk (bf16 packing jobs of the same call that only later kernels read),
// the reduce launch also runs them; without the fused pass they are
// launched first on their own.
struct PackBatchArgs;
hipError_t launch_rowcol(bool bf16, const ColProjArgs& c, const RowProjArgs& r, float* rpartial, hipStream_t st,
                         const PackBatchArgs* pk = nullptr);
// Only the reduce of a fused rowproj: r's outputs from nb column-block partials [nb, T, 16].
hipError_t launch_rowproj_reduce(const RowProjArgs& r, const float* rpartial, int nb, hipStream_t st);
int64_t rowcol_partial_floats(int64_t T, int64_t K);
// partial-buffer floats the bf16 colproj needs for (T, K, R)
int64_t colproj_partial_floats(int64_t T, int64_t K, int R);
int colproj_nchunk(int64_t T, int64_t K);

// Up to three rowcol passes (gradients of the same T, e.g. dQ, dK, dV) in
// one launch plus one launch of both reduces.  Segment s has its own
// scratch: c[s].rpartial [ceil(K_s / 256), T, 16] and c[s].partial
// [nchunk, K_s, 16] fp32, nchunk = rowcol_batch_nchunk(T, K, n) for all
// segments.  Cases launch_rowcol would not fuse, or T = 0, run launch_rowcol
// per segment with the same scratch.
struct RowColBatch {
  ColProjArgs c[3];
  RowProjArgs r[3];
  int32_t kb0[4];  // first column block of each segment; kb0[n] = all blocks
  int32_t n;
  int32_t nx;  // reduce launch only: c[n .. n + nx - 1] are colproj reduces without a rowproj
};
hipError_t launch_rowcol_batch(bool bf16, const ColProjArgs* c, const RowProjArgs* r, int n, hipStream_t st,
                               const PackBatchArgs* pk = nullptr);
// Only the reduces of a rowcol batch whose partials another kernel wrote
// (bf16, r[s].R <= 16): segment s's colproj outputs from c[s].nchunk slices
// c[s].partial [nchunk, K_s, 16] and its rowproj outputs from ceil(K_s / 256)
// slices c[s].rpartial [., T, 16]; in the same launch, the nx colproj reduces
// xc (as launch_colproj_reduce); n + nx <= 3.
hipError_t launch_rowcol_batch_reduce(const ColProjArgs* c, const RowProjArgs* r, int n, const ColProjArgs* xc,
                                      int nx, hipStream_t st);
int rowcol_batch_nchunk(int64_t T, const int64_t* K, int n);
// floats of segment s's colproj partial in a batch
int64_t rowcol_batch_partial_floats(int64_t T, const int64_t* K, int n, int s);

// ---------------------------------------------------------------------------
// Packing of the adapter operands in the layout the kernels read.  A job
// builds the operand of a LoRA K tile over vcols virtual columns and RL rows
// of K: for part descriptors (v0, nv, k0, w, src, ld, nn),
//   value(v0 + n, k0 + i) = nn ? src[i*ld + n] : src[n*ld + i]  (n < nv, i < w),
// everything else 0; stored [vcols, RL] (K-contiguous) or, with kmajor,
// [RL, vcols].  The K-contiguous concatenation [A_0 | A_1 | ...]^T of adapters
// A_q [K, w] is the kmajor job with vcols = K and part q = (0, K, q*w, w, A_q, w, 0).
// All jobs of a call run in one launch.
// ---------------------------------------------------------------------------
struct PackPart {
  const void* src;
  int64_t ld;
  int64_t v0, nv;
  int32_t k0, w, nn, pad_;
};
struct PackLoraArgs {
  void* out;
  int64_t vcols;
  int32_t RL, nparts;
  int32_t kmajor;
  // kmajor operands of NF4 forward (NN) GEMMs: within every 8 columns, column
  // position q holds virtual column 2q (q < 4) or 2(q - 4) + 1, the order in
  // which those GEMMs decode the weight tile (vcols a multiple of 8)
  int32_t perm8;
  PackPart part[6];
};
struct PackBatchArgs {
  PackLoraArgs job[6];
  int32_t njobs;
};
hipError_t launch_pack_batch(bool bf16, const PackBatchArgs& b, hipStream_t st);
hipError_t launch_zero(void* p, int64_t bytes, hipStream_t st);

// fp32 -> bf16 (round to nearest even) of up to six arrays in one launch: the
// adapter cast of the fp32 LoRA-gradient mode.
struct CastSeg {
  const float* src;
  uint16_t* dst;
  int64_t n;
};
struct CastArgs {
  CastSeg seg[6];
  int32_t nseg;
};
hipError_t launch_cast_bf16(const CastArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------
// NF4 kernels.
// ---------------------------------------------------------------------------
hipError_t launch_nf4_quantize(const void* W, int64_t numel, bool bf16, uint8_t* codes,
                               int8_t* q8, float* s2, float* mu, void* ws, hipStream_t st);
size_t nf4_quantize_ws_bytes(int64_t numel);
hipError_t launch_nf4_dequant(const uint8_t* codes, const int8_t* q8, const float* s2,
                              const float* mu, int64_t numel, void* out, bool bf16,
                              hipStream_t st);
hipError_t launch_nf4_unpack(const uint8_t* codes, int64_t numel, uint8_t* out, hipStream_t st);
extern const float kNF4Levels[16];

}  // namespace lora
