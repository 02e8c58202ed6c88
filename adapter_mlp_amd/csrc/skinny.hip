// Rank-r products of the LoRA projections and the small packing kernels.
//
// rowproj   Out[t, j] = sum_k Z[t, k] Bt[j, k]      (T x R, R <= 64)
//   the adapter inputs U = X A (with Bt = A^T) and the hoisted
//   P = dZ B^T (with Bt = B) of the unsloth backward hunks: every P is formed
//   once and then feeds both the A-gradient and the input gradient.
// colproj   Out[k, j] = sum_t Z[t, k] P[t, j]       (K x R, reduction over T)
//   the adapter gradients dA = s X^T P and dB = s U^T dZ (stored transposed).
//
// Both are bound by streaming Z ([T, K] bf16) from HBM once.  The bf16
// versions move Z in 1 KB global-to-LDS loads through a ring of LDS slots
// several steps deep (enough bytes in flight per CU to cover HBM latency),
// and feed v_mfma_f32_16x16x32_bf16 from LDS: row-contiguous operands with
// ds_read_b128, the T-contiguous operands of colproj with the transposing
// ds_read_b64_tr_b16.  Reductions are deterministic: fixed wave order in LDS
// for rowproj, per-chunk partials summed in ascending chunk order for colproj.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace lora {
namespace {

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// ---------------------------------------------------------------------------
// rowproj, bf16.  Block = 32 rows of Z over all of K, 8 wavefronts.  Per
// 256-column chunk, Z [32 x 256] and Bt [16 NJ x 256] land in one ring slot;
// wavefront w multiplies the chunk's K step w (32 columns) into
// acc[row block][column block]; the eight partial sums are added in fixed
// order at the end.  Slot rows are 512 bytes; 16-byte chunk c of row r
// is stored at c ^ (r & 15), so the 16 rows of a fragment read hit 16
// different bank groups.
// ---------------------------------------------------------------------------
template <int NJ>
struct RowProjCfg {
  static constexpr int NW = 8;                  // wavefronts per block (one K step of 8 each)
  static constexpr int ZB = 32 * 512;          // Z bytes per slot
  static constexpr int BB = NJ * 16 * 512;     // Bt bytes per slot
  static constexpr int SB = ZB + BB;
  static constexpr int NST = NJ == 1 ? 6 : NJ == 2 ? 5 : NJ == 3 ? 4 : 3;
  static constexpr int ZPW = 16 / NW;          // Z blocks per wavefront and chunk
  static constexpr int BPW = 8 * NJ / NW;      // Bt blocks per wavefront and chunk
  static constexpr int D = ZPW + BPW;          // loads per wavefront and chunk
  static constexpr int KPW = 8 / NW;           // K steps per wavefront and chunk
};

template <int D, int K>
__device__ __forceinline__ void wait_steps_after(int after) {
  // vmcnt(D * after) for after = 0 .. K (compile-time immediates)
  if constexpr (K > 0) {
    if (after >= K) {
      wait_vmcnt<D * K>();
      return;
    }
    wait_steps_after<D, K - 1>(after);
  } else {
    wait_vmcnt<0>();
  }
}

template <int NJ>
__global__ __launch_bounds__(RowProjCfg<NJ>::NW * 64) void rowproj_bf16_kernel(const RowProjArgs a) {
  using C = RowProjCfg<NJ>;
  __shared__ __attribute__((aligned(1024))) char ring[C::NST * C::SB];
  lds_char* const lds = (lds_char*)ring;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int64_t rows = a.T - t0 < 32 ? a.T - t0 : 32;
  const int nch = (int)((a.K + 255) / 256);
  const uint32_t ldz2 = (uint32_t)(a.ldz * 2), ldb2 = (uint32_t)(a.ldb * 2);
  // rows past T and adapter rows past R read as zero
  const i32x4 rz = rsrc_words(static_cast<const char*>(a.Z) + t0 * a.ldz * 2, rows * a.ldz * 2);
  const i32x4 rb = rsrc_words(a.Bt, (int64_t)a.R * a.ldb * 2);

  // load blocks of this wavefront: Z blocks ZPW w .. (rows 2q, 2q+1), Bt
  // blocks BPW w .. (rows 2q', 2q'+1); lane -> row q*2 + lane/32, chunk lane%32
  const int hrow = lane >> 5, pc = lane & 31;
  uint32_t zoff[C::ZPW], boff[C::BPW];
#pragma unroll
  for (int i = 0; i < C::ZPW; ++i) {
    const int row = 2 * (C::ZPW * w + i) + hrow;
    zoff[i] = (uint32_t)row * ldz2 + (uint32_t)((pc ^ (row & 15)) * 16);
  }
#pragma unroll
  for (int i = 0; i < C::BPW; ++i) {
    const int row = 2 * (C::BPW * w + i) + hrow;
    boff[i] = (uint32_t)row * ldb2 + (uint32_t)((pc ^ (row & 15)) * 16);
  }
  // Block b walks the K chunks starting at chunk b mod nch, so that blocks
  // running together read different column ranges of Z's rows rather than
  // all the same one (measured: the pass over X at the Llama-3-8B MLP shape
  // 24 -> 20 us).  The sum order over chunks is fixed per block.
  const int rot = nch > 0 ? (int)(blockIdx.x % (unsigned)nch) : 0;
  auto cmap = [&](int c) {
    const int x = c + rot;
    return x >= nch ? x - nch : x;
  };
  auto issue = [&](int c, int slot) {
    const uint32_t base = lds_addr(lds) + slot * C::SB;
    const uint32_t soff = (uint32_t)cmap(c) * 512;
#pragma unroll
    for (int i = 0; i < C::ZPW; ++i) dma16(rz, zoff[i], base + (C::ZPW * w + i) * 1024, soff);
#pragma unroll
    for (int i = 0; i < C::BPW; ++i) dma16(rb, boff[i], base + C::ZB + (C::BPW * w + i) * 1024, soff);
  };

  f32x4 acc[2][NJ];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NJ; ++nb) acc[mb][nb] = f32x4{0, 0, 0, 0};
  // fragment chunk of K step ks (0..7) for this lane: 4 ks + lane / 16, stored
  // at that ^ (lane & 15) in rows mb*16 + lane%16 and nb*16 + lane%16
  const int rl = lane & 15;
  auto compute = [&](int c, int slot) {
    const lds_char* zs = lds + slot * C::SB;
    const lds_char* bs = zs + C::ZB;
#pragma unroll
    for (int i = 0; i < C::KPW; ++i) {
      const int ks = C::KPW * w + i;
      if ((int64_t)cmap(c) * 256 + ks * 32 >= a.K) continue;  // K tail (uniform)
      const int off = ((4 * ks + (lane >> 4)) ^ rl) * 16;
      bf16x8 za[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        za[mb] = __builtin_bit_cast(bf16x8, lds_read16(zs + (mb * 16 + rl) * 512 + off));
#pragma unroll
      for (int nb = 0; nb < NJ; ++nb) {
        const bf16x8 bb = __builtin_bit_cast(bf16x8, lds_read16(bs + (nb * 16 + rl) * 512 + off));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za[mb], bb, acc[mb][nb], 0, 0, 0);
      }
    }
  };

  const int pre = nch < C::NST - 1 ? nch : C::NST - 1;
  for (int c = 0; c < pre; ++c) issue(c, c);
  for (int c = 0; c < nch; ++c) {
    const int after = (nch - 1 - c) < (C::NST - 2) ? (nch - 1 - c) : (C::NST - 2);
    wait_steps_after<C::D, C::NST - 2>(after);  // chunk c of this wavefront has landed
    __syncthreads();                            // everyone's has; chunk c-1's slot is free
    if (c + C::NST - 1 < nch) issue(c + C::NST - 1, (c + C::NST - 1) % C::NST);
    compute(c, c % C::NST);
  }
  __syncthreads();

  // acc[mb][nb][v] = Out[t0 + 16 mb + 4 (lane >> 4) + v, 16 nb + lane % 16] (K share of wavefront w)
  float* red = reinterpret_cast<float*>(ring);  // [NW][32][16 NJ]
  constexpr int RW = NJ * 16;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NJ; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(w * 32 + mb * 16 + 4 * (lane >> 4) + v) * RW + nb * 16 + rl] = acc[mb][nb][v];
  __syncthreads();
  const int R2 = a.R2 > a.R ? a.R2 : a.R;
  for (int e = tid; e < 32 * R2; e += C::NW * 64) {
    const int r = e / R2, j = e % R2;
    const int64_t t = t0 + r;
    if (t >= a.T) continue;
    float v = 0.0f;
    if (j < a.R) {
#pragma unroll
      for (int q = 0; q < C::NW; ++q) v += red[(q * 32 + r) * RW + j];  // fixed order
    }
    if (a.out1 && j < a.R) static_cast<uint16_t*>(a.out1)[t * a.ld1 + a.off1 + j] = (uint16_t)f2bf(v);
    if (a.out2) {
      const float sc = j < a.R ? a.scales[j / a.seg_w] : 0.0f;
      static_cast<uint16_t*>(a.out2)[t * a.ld2 + j] = (uint16_t)f2bf(sc * v);
    }
  }
}

__global__ void rowproj_f32_kernel(const RowProjArgs a) {
  const int R2 = a.R2 > a.R ? a.R2 : a.R;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.T * R2) return;
  const int64_t t = e / R2;
  const int j = (int)(e % R2);
  float v = 0.0f;
  if (j < a.R) {
    const float* z = static_cast<const float*>(a.Z) + t * a.ldz;
    const float* b = static_cast<const float*>(a.Bt) + (int64_t)j * a.ldb;
    for (int64_t k = 0; k < a.K; ++k) v = fmaf(z[k], b[k], v);
  }
  if (a.out1 && j < a.R) static_cast<float*>(a.out1)[t * a.ld1 + a.off1 + j] = v;
  if (a.out2) {
    const float sc = j < a.R ? a.scales[j / a.seg_w] : 0.0f;
    static_cast<float*>(a.out2)[t * a.ld2 + j] = sc * v;
  }
}

// ---------------------------------------------------------------------------
// colproj, bf16.  Block = 256 columns of Z (k) x one chunk of T (a multiple
// of 32 rows), 4 wavefronts.  Per 32-row step, Z [32 x 256] and P [32 x PW]
// land in one ring slot; wavefront w owns columns 64 w .. 64 w + 63 (four
// 16-row MFMA blocks of Z^T) and accumulates over the chunk.  Both operands
// are T-contiguous in the MFMA, so they are read with ds_read_b64_tr_b16:
// lane s of a read points at row 8 g + 4 h + (s & 15) / 4 (g = s / 16,
// h = 0, 1) and 4 columns at 4 (s & 3).  Z slot rows are 512 bytes, 16-byte
// chunk c of row t stored at c ^ zswz(t); the 16 rows x 32 bytes of one
// transposing read then fall on every bank group exactly twice.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int zswz(int t) { return 2 * ((t & 3) + 4 * ((t >> 3) & 1)); }

template <int NJ>
struct ColProjCfg {
  static constexpr int PW = NJ == 3 ? 64 : NJ * 16;  // staged P columns
  static constexpr int ZB = 32 * 512;
  static constexpr int PB = 32 * PW * 2;             // 1, 2 or 4 KB
  static constexpr int NPB = PB / 1024;              // P load blocks per step
  static constexpr int SB = ZB + PB;
  static constexpr int NST = 4;
};

// With ROW, the block also forms a rowproj over its 256 columns: Out[t, j] =
// sum_k Z[t, k] Bt[j, k] for every 32-row step, written as that column
// block's partial.  The Bt slice [16 x 256] is loaded once into LDS (rows of
// 512 bytes, chunk c of row j at c ^ j) and from there into registers; per
// step, wavefronts 0, 1 (even steps) or 2, 3 (odd steps) each take one
// 16-row half with 8 16x16x32 MFMAs, reading Z K-contiguously from the slot.
// Column block kb of a (the block's 256 columns of Z), row chunk blockIdx.y.
template <int NJ, bool ROW>
__device__ __forceinline__ void colproj_body(const ColProjArgs& a, int64_t rows_per_chunk, int64_t kb) {
  using C = ColProjCfg<NJ>;
  constexpr int BTB = ROW ? 8192 : 0;  // Bt slice after the ring
  constexpr int RSB = ROW ? 2048 : 0;  // then the rowproj output staging, 1 KB per wavefront of a step
  __shared__ __attribute__((aligned(1024))) char ring[C::NST * C::SB + BTB + RSB];
  lds_char* const lds = (lds_char*)ring;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t k0 = kb * 256;
  const int64_t c = blockIdx.y;
  const int64_t tbeg = c * rows_per_chunk;
  const int64_t tend = tbeg + rows_per_chunk < a.T ? tbeg + rows_per_chunk : a.T;
  const int nsteps = (int)((tend - tbeg + 31) / 32);
  const uint32_t ldz2 = (uint32_t)(a.ldz * 2), ldp2 = (uint32_t)(a.ldp * 2);
  // rows past T read as zero; columns past K (last column block) only reach
  // outputs k >= K, which are not stored
  const i32x4 rz = rsrc_words(static_cast<const char*>(a.Z) + (tbeg * a.ldz + k0) * 2,
                              (a.T - tbeg) * a.ldz * 2 - k0 * 2);
  const i32x4 rp = rsrc_words(static_cast<const char*>(a.P) + tbeg * a.ldp * 2, (a.T - tbeg) * a.ldp * 2);

  // Z blocks 4w..4w+3 (rows 2q, 2q+1; lane -> row 2q + lane/32, chunk lane%32);
  // P block w if w < NPB (rows 32/NPB per block, PW/8 chunks per row)
  const int hrow = lane >> 5, pc = lane & 31;
  uint32_t zoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 2 * (4 * w + i) + hrow;
    zoff[i] = (uint32_t)row * ldz2 + (uint32_t)((pc ^ zswz(row)) * 16);
  }
  constexpr int PCH = C::PW / 8;  // 16-byte chunks per P row
  const int prow = w * (64 / PCH) + lane / PCH;
  const uint32_t poff = (uint32_t)prow * ldp2 + (uint32_t)((lane % PCH) * 16);
  const bool pload = w < C::NPB;
  auto issue = [&](int s, int slot) {
    const uint32_t base = lds_addr(lds) + slot * C::SB;
    const uint32_t zs = (uint32_t)s * 32 * ldz2, ps = (uint32_t)s * 32 * ldp2;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rz, zoff[i], base + (4 * w + i) * 1024, zs);
    if (pload) dma16(rp, poff, base + C::ZB + w * 1024, ps);
  };

  f32x4 acc[4][NJ];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nb = 0; nb < NJ; ++nb) acc[mi][nb] = f32x4{0, 0, 0, 0};
  // transposing-read addresses (bytes in a slot), read h adds 4 rows
  const int g = lane >> 4, i15 = lane & 15;
  const int tr = 8 * g + (i15 >> 2);  // row of read h = 0
  int zaddr[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int col = 16 * (4 * w + mi) + 4 * (i15 & 3);
    zaddr[mi] = tr * 512 + (((col >> 3) ^ zswz(tr)) * 16) + (col & 7) * 2;
  }
  auto compute = [&](int slot) {
    const lds_char* zs = lds + slot * C::SB;
    const lds_char* ps = zs + C::ZB;
    bf16x8 pb[NJ];
#pragma unroll
    for (int nb = 0; nb < NJ; ++nb) pb[nb] = lds_read_tr8(ps + tr * (C::PW * 2) + (16 * nb + 4 * (i15 & 3)) * 2, 4 * C::PW * 2);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const bf16x8 za = lds_read_tr8(zs + zaddr[mi], 4 * 512);
#pragma unroll
      for (int nb = 0; nb < NJ; ++nb)
        acc[mi][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za, pb[nb], acc[mi][nb], 0, 0, 0);
    }
  };

  // ---- fused rowproj (ROW) ----
  bf16x8 btf[ROW ? 8 : 1];
  auto row_step = [&](int s, int slot) {
    if constexpr (ROW) {
      if ((w >> 1) != (s & 1)) return;  // two wavefronts per step
      const int rb = w & 1;             // 16-row half of the step
      const lds_char* zs = lds + slot * C::SB;
      const int r = rb * 16 + (lane & 15);
      f32x4 acc_r = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int cz = 4 * ks + (lane >> 4);
        const bf16x8 za = __builtin_bit_cast(bf16x8, lds_read16(zs + r * 512 + ((cz ^ zswz(r)) * 16)));
        acc_r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za, btf[ks], acc_r, 0, 0, 0);
      }
      // acc_r[v] = Out[row rb * 16 + 4 (lane >> 4) + v of the step, j = lane % 16].  The 16 x 16
      // block is staged row-major in LDS and stored as 16-byte pieces: rows t .. t + 15 of the
      // partial are 1 KB of consecutive floats, written by one store per lane.  (Four 4-byte
      // stores per lane, each scattering 64-byte pieces over four rows, cost the pass about a
      // fifth of its time.)  The other pair of wavefronts reuses this staging in the next step,
      // after that step's barrier.
      float* const stg = reinterpret_cast<float*>(ring + C::NST * C::SB + BTB) + rb * 256;
#pragma unroll
      for (int v = 0; v < 4; ++v) stg[(4 * (lane >> 4) + v) * 16 + (lane & 15)] = acc_r[v];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wavefront's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      const f32x4 o = *reinterpret_cast<const f32x4*>(stg + 4 * lane);  // row lane / 4, j = 4 (lane % 4) ..
      const int64_t t = tbeg + 32 * (int64_t)s + rb * 16 + (lane >> 2);
      if (t < tend) *reinterpret_cast<f32x4*>(a.rpartial + (kb * a.T + t) * 16 + 4 * (lane & 3)) = o;
    }
  };

  if constexpr (ROW) {
    // Bt slice: rows past R1 read zero; two 1 KB loads per wavefront (rows 2q, 2q+1)
    const i32x4 rbt = rsrc_words(static_cast<const char*>(a.Bt) + k0 * 2, (int64_t)a.R1 * a.ldb * 2 - k0 * 2);
    const uint32_t ldb2 = (uint32_t)(a.ldb * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 2 * (2 * w + i) + hrow;
      dma16(rbt, (uint32_t)row * ldb2 + (uint32_t)((pc ^ row) * 16), lds_addr(lds) + C::NST * C::SB + (2 * w + i) * 1024);
    }
  }
  const int pre = nsteps < C::NST - 1 ? nsteps : C::NST - 1;
  for (int s = 0; s < pre; ++s) issue(s, s);
  for (int s = 0; s < nsteps; ++s) {
    const int after = (nsteps - 1 - s) < (C::NST - 2) ? (nsteps - 1 - s) : (C::NST - 2);
    if (pload) wait_steps_after<5, C::NST - 2>(after);
    else wait_steps_after<4, C::NST - 2>(after);
    __syncthreads();
    if constexpr (ROW) {
      if (s == 0) {  // the Bt slice (loaded before step 0) is in: fragments for all 8 K steps;
        // columns past K (last block) are zeroed, whole fragments since K is a multiple of 64
        const lds_char* bs = lds + C::NST * C::SB;
        const int j = lane & 15;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int cb = 4 * ks + (lane >> 4);
          const u32x4 v = lds_read16(bs + j * 512 + ((cb ^ j) * 16));
          const bool in = k0 + 8 * cb < a.K;
          btf[ks] = __builtin_bit_cast(bf16x8, in ? v : u32x4{0, 0, 0, 0});
        }
      }
    }
    if (s + C::NST - 1 < nsteps) issue(s + C::NST - 1, (s + C::NST - 1) % C::NST);
    compute(s % C::NST);
    row_step(s, s % C::NST);
  }

  // acc[mi][nb][v] = Out[k0 + 16 (4w + mi) + 4 (lane >> 4) + v, 16 nb + lane % 16]
  const int Rp = NJ * 16;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nb = 0; nb < NJ; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t k = k0 + 16 * (4 * w + mi) + 4 * (lane >> 4) + v;
        if (k < a.K) a.partial[(c * a.K + k) * Rp + nb * 16 + i15] = acc[mi][nb][v];
      }
}

template <int NJ, bool ROW>
__global__ __launch_bounds__(256) void colproj_bf16_kernel(const ColProjArgs a, int64_t rows_per_chunk) {
  colproj_body<NJ, ROW>(a, rows_per_chunk, blockIdx.x);
}

// Fused rank-r passes over up to three gradients of the same T in one launch:
// the column blocks of segment s are kb0[s] .. kb0[s + 1] - 1.
__global__ __launch_bounds__(256) void rowcol_batch_kernel(const RowColBatch b, int64_t rows_per_chunk) {
  int s = 0;
  for (int i = 1; i < b.n; ++i)
    if ((int)blockIdx.x >= b.kb0[i]) s = i;
  colproj_body<1, true>(b.c[s], rows_per_chunk, (int64_t)blockIdx.x - b.kb0[s]);
}

__device__ __forceinline__ void colproj_store(const ColProjArgs& a, bool bf16, int64_t k, int j, float v) {
  const int q = j / a.seg_w, jj = j % a.seg_w;
  const float o = a.scales[q] * v;
  const int64_t idx = a.transposed ? (int64_t)jj * a.K + k : k * a.seg_w + jj;
  if (bf16) static_cast<uint16_t*>(a.dest[q])[idx] = (uint16_t)f2bf(o);
  else static_cast<float*>(a.dest[q])[idx] = o;
}

// dest = scales * (sum over the a.nchunk slices of partial [nchunk, K, Rp]).
// A block takes 64 outputs of 4 consecutive columns j of one k (R is a
// multiple of 4 in the bf16 path; the 4 never straddle two adapters since
// seg_w is a multiple of 8) and splits the slices into 4 contiguous ranges,
// one per group of 64 threads: 16-byte loads on consecutive addresses.  Each
// range is summed in ascending order and the 4 range sums are added in
// ascending order, so the result does not depend on the launch.
constexpr int RED_PARTS = 4;
__device__ __forceinline__ f32x4 sum_slices(const float* src, int64_t stride, int b0, int b1) {
  f32x4 v = f32x4{0, 0, 0, 0};
  int b = b0;
  for (; b + 4 <= b1; b += 4) {
    const f32x4 p0 = *reinterpret_cast<const f32x4*>(src + (b + 0) * stride);
    const f32x4 p1 = *reinterpret_cast<const f32x4*>(src + (b + 1) * stride);
    const f32x4 p2 = *reinterpret_cast<const f32x4*>(src + (b + 2) * stride);
    const f32x4 p3 = *reinterpret_cast<const f32x4*>(src + (b + 3) * stride);
    v += p0;
    v += p1;
    v += p2;
    v += p3;
  }
  for (; b < b1; ++b) v += *reinterpret_cast<const f32x4*>(src + b * stride);
  return v;
}

__device__ __forceinline__ void colproj_reduce_body(const ColProjArgs& a, int Rp, int64_t bx) {
  __shared__ f32x4 part[RED_PARTS][64];
  const int RQ = a.R / 4;
  const int pq = threadIdx.x >> 6, o = threadIdx.x & 63;
  const int64_t e = bx * 64 + o;
  const bool live = e < a.K * RQ;
  const int64_t k = live ? e / RQ : 0;
  const int j0 = live ? (int)(e % RQ) * 4 : 0;
  if (live)
    part[pq][o] = sum_slices(a.partial + k * Rp + j0, a.K * Rp, (int)((int64_t)pq * a.nchunk / RED_PARTS),
                             (int)((int64_t)(pq + 1) * a.nchunk / RED_PARTS));
  __syncthreads();
  if (pq != 0 || !live) return;
  f32x4 v = part[0][o];
#pragma unroll
  for (int q = 1; q < RED_PARTS; ++q) v += part[q][o];
#pragma unroll
  for (int q = 0; q < 4; ++q) colproj_store(a, a.out_f32 == 0, k, j0 + q, v[q]);
}
__global__ __launch_bounds__(256) void colproj_reduce_kernel(const ColProjArgs a, int Rp) {
  colproj_reduce_body(a, Rp, blockIdx.x);
}

__global__ void colproj_f32_kernel(const ColProjArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.K * a.R) return;
  const int64_t k = e / a.R;
  const int j = (int)(e % a.R);
  const float* z = static_cast<const float*>(a.Z);
  const float* p = static_cast<const float*>(a.P);
  float v = 0.0f;
  for (int64_t t = 0; t < a.T; ++t) v = fmaf(z[t * a.ldz + k], p[t * a.ldp + j], v);
  colproj_store(a, false, k, j, v);
}

// ---------------------------------------------------------------------------
// Packing.
// ---------------------------------------------------------------------------
// Every pack job of a call in one launch (blockIdx.y = job).  Threads walk
// each output in storage order, so the stores are coalesced; the sources
// (adapters, at most a few MB) are read from L2.
template <typename E>
__device__ __forceinline__ void pack_job(const PackLoraArgs& a, uint32_t first, uint32_t stride) {
  // 32-bit index arithmetic (a 64-bit division per element dominated the
  // kernel); the launchers check that every job has fewer than 2^31 elements
  const uint32_t vc = (uint32_t)a.vcols, rl = (uint32_t)a.RL, n = vc * rl;
  for (uint32_t o = first; o < n; o += stride) {
    uint32_t v = a.kmajor ? o % vc : o / rl;
    const uint32_t kk = a.kmajor ? o / vc : o % rl;
    if (a.perm8) v = (v & ~7u) | ((v & 3u) << 1) | ((v >> 2) & 1u);
    E val = E(0);
    for (int p = 0; p < a.nparts; ++p) {
      const PackPart& q = a.part[p];
      const uint32_t nn = v - (uint32_t)q.v0, i = kk - (uint32_t)q.k0;  // wrap past the part's range
      if (nn < (uint32_t)q.nv && i < (uint32_t)q.w) {
        const E* src = static_cast<const E*>(q.src);
        val = q.nn ? src[(size_t)i * q.ld + nn] : src[(size_t)nn * q.ld + i];
      }
    }
    static_cast<E*>(a.out)[o] = val;
  }
}
template <typename E>
__global__ void pack_batch_kernel(const PackBatchArgs b) {
  pack_job<E>(b.job[blockIdx.y], blockIdx.x * blockDim.x + threadIdx.x, gridDim.x * blockDim.x);
}

__global__ void cast_bf16_kernel(const CastArgs a) {
  const CastSeg& q = a.seg[blockIdx.y];
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < q.n; e += (int64_t)gridDim.x * blockDim.x)
    q.dst[e] = (uint16_t)f2bf(q.src[e]);
}

__global__ void zero_kernel(uint32_t* p, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) p[e] = 0u;
}

inline unsigned nblk(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }

}  // namespace

namespace {
// chunks of T for a colproj grid of kblocks column blocks
int nchunk_for(int64_t T, int64_t kblocks) {
  const int64_t steps = (T + 31) / 32;
  if (steps == 0) return 0;
  // at most one round of two blocks per CU: a partial second round would run
  // its few blocks while most CUs idle
  int64_t want = 512 / kblocks;
  if (want < 1) want = 1;
  return (int)(want < steps ? want : steps);
}
// the chunk count after rounding the chunk to whole 32-row steps
int nchunk_rounded(int64_t T, int nchunk, int64_t* rows_per_chunk) {
  const int64_t steps = (T + 31) / 32;
  const int64_t spc = (steps + nchunk - 1) / nchunk;
  *rows_per_chunk = spc * 32;
  return (int)((T + *rows_per_chunk - 1) / *rows_per_chunk);
}
}  // namespace

int colproj_nchunk(int64_t T, int64_t K) { return nchunk_for(T, (K + 255) / 256); }

int rowcol_batch_nchunk(int64_t T, const int64_t* K, int n) {
  int64_t kb = 0;
  for (int i = 0; i < n; ++i) kb += (K[i] + 255) / 256;
  return nchunk_for(T, kb);
}
int64_t rowcol_batch_partial_floats(int64_t T, const int64_t* K, int n, int s) {
  return (int64_t)rowcol_batch_nchunk(T, K, n) * K[s] * 16;
}

int64_t colproj_partial_floats(int64_t T, int64_t K, int R) {
  const int Rp = ((R + 15) / 16) * 16;
  return (int64_t)colproj_nchunk(T, K) * K * Rp;
}

hipError_t launch_rowproj(bool bf16, const RowProjArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  if (!bf16) {
    const int R2 = a.R2 > a.R ? a.R2 : a.R;
    hipLaunchKernelGGL(rowproj_f32_kernel, dim3(nblk(a.T * R2, 256)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid(nblk(a.T, 32));
  switch ((a.R + 15) / 16) {
    case 1: hipLaunchKernelGGL(rowproj_bf16_kernel<1>, grid, dim3(RowProjCfg<1>::NW * 64), 0, st, a); break;
    case 2: hipLaunchKernelGGL(rowproj_bf16_kernel<2>, grid, dim3(RowProjCfg<2>::NW * 64), 0, st, a); break;
    case 3: hipLaunchKernelGGL(rowproj_bf16_kernel<3>, grid, dim3(RowProjCfg<3>::NW * 64), 0, st, a); break;
    default: hipLaunchKernelGGL(rowproj_bf16_kernel<4>, grid, dim3(RowProjCfg<4>::NW * 64), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_colproj_reduce(const ColProjArgs& a, hipStream_t st) {
  if (a.K * a.R == 0) return hipSuccess;
  hipLaunchKernelGGL(colproj_reduce_kernel, dim3(nblk(a.K * (a.R / 4), 64)), dim3(256), 0, st, a, 16);
  return hipGetLastError();
}

hipError_t launch_colproj(bool bf16, const ColProjArgs& a0, hipStream_t st) {
  ColProjArgs a = a0;
  if (!bf16) {
    if (a.K * a.R == 0) return hipSuccess;
    hipLaunchKernelGGL(colproj_f32_kernel, dim3(nblk(a.K * a.R, 256)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const int NJ = (a.R + 15) / 16;
  a.nchunk = colproj_nchunk(a.T, a.K);
  if (a.nchunk > 0) {
    const int64_t steps = (a.T + 31) / 32;
    const int64_t steps_per_chunk = (steps + a.nchunk - 1) / a.nchunk;
    const int64_t rows_per_chunk = steps_per_chunk * 32;
    a.nchunk = (int)((a.T + rows_per_chunk - 1) / rows_per_chunk);
    const dim3 grid((unsigned)((a.K + 255) / 256), (unsigned)a.nchunk);
    if (a.rpartial != nullptr) {  // fused rowproj (launch_rowcol): NJ == 1
      hipLaunchKernelGGL((colproj_bf16_kernel<1, true>), grid, dim3(256), 0, st, a, rows_per_chunk);
    } else {
      switch (NJ) {
        case 1: hipLaunchKernelGGL((colproj_bf16_kernel<1, false>), grid, dim3(256), 0, st, a, rows_per_chunk); break;
        case 2: hipLaunchKernelGGL((colproj_bf16_kernel<2, false>), grid, dim3(256), 0, st, a, rows_per_chunk); break;
        case 3: hipLaunchKernelGGL((colproj_bf16_kernel<3, false>), grid, dim3(256), 0, st, a, rows_per_chunk); break;
        default: hipLaunchKernelGGL((colproj_bf16_kernel<4, false>), grid, dim3(256), 0, st, a, rows_per_chunk); break;
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(colproj_reduce_kernel, dim3(nblk(a.K * (a.R / 4), 64)), dim3(256), 0, st, a, NJ * 16);
  return hipGetLastError();
}

namespace {
// Out[t, j] of a fused rowproj: the column blocks' partials [nb, T, 16]
// summed, then written as the rowproj kernel writes it.  A block takes 16
// rows x 4 quads of columns (j < 16) and splits the blocks into 4 contiguous
// ranges as in colproj_reduce_kernel (ascending within a range, ranges added
// in ascending order); the quad-0 threads also write the zero padding of
// out2 past 16.
__device__ __forceinline__ void rowproj_reduce_body(const RowProjArgs& a, const float* rpartial, int nb, int64_t bx) {
  __shared__ f32x4 part[RED_PARTS][64];
  const int R2 = a.R2 > a.R ? a.R2 : a.R;
  const int pq = threadIdx.x >> 6, o = threadIdx.x & 63;
  const int64_t e = bx * 64 + o;
  const bool live = e < a.T * 4;
  const int64_t t = e >> 2;
  const int j0 = (o & 3) * 4;
  if (live)
    part[pq][o] = j0 < a.R ? sum_slices(rpartial + t * 16 + j0, a.T * 16, (int)((int64_t)pq * nb / RED_PARTS),
                                        (int)((int64_t)(pq + 1) * nb / RED_PARTS))
                           : f32x4{0, 0, 0, 0};
  __syncthreads();
  if (pq != 0 || !live) return;
  f32x4 v = part[0][o];
#pragma unroll
  for (int q = 1; q < RED_PARTS; ++q) v += part[q][o];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = j0 + q;
    if (j >= R2) break;
    const float x = j < a.R ? v[q] : 0.0f;
    if (a.out1 && j < a.R) static_cast<uint16_t*>(a.out1)[t * a.ld1 + a.off1 + j] = (uint16_t)f2bf(x);
    if (a.out2) {
      const float sc = j < a.R ? a.scales[j / a.seg_w] : 0.0f;
      static_cast<uint16_t*>(a.out2)[t * a.ld2 + j] = (uint16_t)f2bf(sc * x);
    }
  }
  if (a.out2 && j0 == 0)
    for (int j = 16; j < R2; ++j) static_cast<uint16_t*>(a.out2)[t * a.ld2 + j] = 0;
}
__global__ __launch_bounds__(256) void rowproj_reduce_kernel(const RowProjArgs a, const float* rpartial, int nb) {
  rowproj_reduce_body(a, rpartial, nb, blockIdx.x);
}
// Both reduces of a rowcol batch: blockIdx.y < n the colproj reduce (dB) of
// segment y, else the rowproj reduce (P) of segment y - n.
__device__ __forceinline__ void rowcol_reduce_part(const RowColBatch& b, int y) {
  if (y < b.n) {
    colproj_reduce_body(b.c[y], 16, blockIdx.x);
  } else if (y < 2 * b.n) {
    const int s = y - b.n;
    rowproj_reduce_body(b.r[s], b.c[s].rpartial, b.kb0[s + 1] - b.kb0[s], blockIdx.x);
  } else {
    colproj_reduce_body(b.c[y - b.n], 16, blockIdx.x);  // the extra colproj reduces
  }
}
__global__ __launch_bounds__(256) void rowcol_batch_reduce_kernel(const RowColBatch b) {
  rowcol_reduce_part(b, blockIdx.y);
}
// The same reduces, and past them (blockIdx.y) the bf16 adapter-packing jobs of
// the same call, which a later kernel reads: one launch instead of two.
__global__ __launch_bounds__(256) void rowcol_batch_reduce_pack_kernel(const RowColBatch b, const PackBatchArgs pk) {
  const int nr = 2 * b.n + b.nx;
  if ((int)blockIdx.y < nr) rowcol_reduce_part(b, blockIdx.y);
  else pack_job<uint16_t>(pk.job[blockIdx.y - nr], blockIdx.x * blockDim.x + threadIdx.x, gridDim.x * blockDim.x);
}
static_assert(sizeof(RowColBatch) + sizeof(PackBatchArgs) <= 4096, "kernel arguments exceed 4 KB");
}  // namespace

int64_t rowcol_partial_floats(int64_t T, int64_t K) { return ((K + 255) / 256) * T * 16; }

// Blocks per job of a pack launch (0: nothing to pack; -1: a job too large).
static int64_t pack_grid_x(const PackBatchArgs& b) {
  int64_t nmax = 0;
  for (int i = 0; i < b.njobs; ++i) nmax = b.job[i].vcols * b.job[i].RL > nmax ? b.job[i].vcols * b.job[i].RL : nmax;
  if (b.njobs <= 0 || nmax == 0) return 0;
  if (nmax >= ((int64_t)1 << 31)) return -1;
  return nblk(nmax, 256) < 2048 ? nblk(nmax, 256) : 2048;
}

hipError_t launch_rowcol(bool bf16, const ColProjArgs& c0, const RowProjArgs& r, float* rpartial, hipStream_t st,
                         const PackBatchArgs* pk) {
  const bool fused = bf16 && rpartial != nullptr && r.R <= 16 && r.Z == c0.Z && r.ldz == c0.ldz && r.T == c0.T &&
                     r.K == c0.K && r.K % 8 == 0 && c0.R <= 16 && c0.T > 0;
  if (!fused) {
    if (pk != nullptr) {
      const hipError_t e = launch_pack_batch(bf16, *pk, st);
      if (e != hipSuccess) return e;
    }
    hipError_t e = launch_rowproj(bf16, r, st);
    if (e != hipSuccess) return e;
    // the plain colproj: a set rpartial would select the fused (R <= 16) kernel
    ColProjArgs c = c0;
    c.rpartial = nullptr;
    return launch_colproj(bf16, c, st);
  }
  // a batch of one: the pass, then both reduces in one launch (the chunking
  // is that of launch_colproj, so the sums are the same)
  ColProjArgs c = c0;
  c.rpartial = rpartial;
  return launch_rowcol_batch(true, &c, &r, 1, st, pk);
}

hipError_t launch_rowcol_batch(bool bf16, const ColProjArgs* c, const RowProjArgs* r, int n, hipStream_t st,
                               const PackBatchArgs* pk) {
  if (n < 1 || n > 3) return hipErrorInvalidValue;
  bool fused = bf16 && c[0].T > 0;
  for (int i = 0; i < n && fused; ++i)
    fused = c[i].rpartial != nullptr && r[i].R <= 16 && r[i].Z == c[i].Z && r[i].ldz == c[i].ldz &&
            r[i].T == c[i].T && r[i].K == c[i].K && r[i].K % 8 == 0 && c[i].R <= 16 && c[i].T == c[0].T;
  if (!fused) {
    if (pk != nullptr) {
      const hipError_t e = launch_pack_batch(bf16, *pk, st);
      if (e != hipSuccess) return e;
    }
    for (int i = 0; i < n; ++i) {
      const hipError_t e = launch_rowcol(bf16, c[i], r[i], c[i].rpartial, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  RowColBatch b{};
  b.n = n;
  int64_t K[3];
  unsigned rx = nblk(c[0].T * 4, 64);  // reduce blocks: the rowproj side
  for (int i = 0; i < n; ++i) {
    K[i] = c[i].K;
    b.kb0[i + 1] = b.kb0[i] + (int32_t)((c[i].K + 255) / 256);
    const unsigned cx = nblk(c[i].K * (c[i].R / 4), 64);
    rx = cx > rx ? cx : rx;
  }
  int64_t rows_per_chunk = 0;
  const int nchunk = nchunk_rounded(c[0].T, rowcol_batch_nchunk(c[0].T, K, n), &rows_per_chunk);
  for (int i = 0; i < n; ++i) {
    b.c[i] = c[i];
    b.c[i].Bt = r[i].Bt;
    b.c[i].ldb = r[i].ldb;
    b.c[i].R1 = r[i].R;
    b.c[i].nchunk = nchunk;
    b.r[i] = r[i];
  }
  const int64_t px = pk != nullptr ? pack_grid_x(*pk) : 0;
  if (px < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rowcol_batch_kernel, dim3((unsigned)b.kb0[n], (unsigned)nchunk), dim3(256), 0, st, b,
                     rows_per_chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (px > 0) {
    const unsigned gx = (unsigned)px > rx ? (unsigned)px : rx;
    hipLaunchKernelGGL(rowcol_batch_reduce_pack_kernel, dim3(gx, (unsigned)(2 * n + pk->njobs)), dim3(256), 0, st, b,
                       *pk);
  } else {
    hipLaunchKernelGGL(rowcol_batch_reduce_kernel, dim3(rx, (unsigned)(2 * n)), dim3(256), 0, st, b);
  }
  return hipGetLastError();
}

hipError_t launch_rowcol_batch_reduce(const ColProjArgs* c, const RowProjArgs* r, int n, const ColProjArgs* xc,
                                      int nx, hipStream_t st) {
  if (n < 1 || nx < 0 || n + nx > 3) return hipErrorInvalidValue;
  RowColBatch b{};
  b.n = n;
  b.nx = nx;
  unsigned rx = nblk(c[0].T * 4, 64);  // reduce blocks: the rowproj side
  for (int i = 0; i < n; ++i) {
    if (r[i].R > 16 || c[i].R > 16 || c[i].T != c[0].T || r[i].T != c[0].T) return hipErrorInvalidValue;
    b.kb0[i + 1] = b.kb0[i] + (int32_t)((c[i].K + 255) / 256);
    const unsigned cx = nblk(c[i].K * (c[i].R / 4), 64);
    rx = cx > rx ? cx : rx;
    b.c[i] = c[i];
    b.r[i] = r[i];
  }
  for (int i = 0; i < nx; ++i) {
    if (xc[i].R > 16) return hipErrorInvalidValue;
    const unsigned cx = nblk(xc[i].K * (xc[i].R / 4), 64);
    rx = cx > rx ? cx : rx;
    b.c[n + i] = xc[i];
  }
  // T = 0 still writes the colproj outputs: sums over no slices, zero
  if (rx == 0) return hipSuccess;
  hipLaunchKernelGGL(rowcol_batch_reduce_kernel, dim3(rx, (unsigned)(2 * n + nx)), dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_rowproj_reduce(const RowProjArgs& r, const float* rpartial, int nb, hipStream_t st) {
  if (r.T == 0) return hipSuccess;
  hipLaunchKernelGGL(rowproj_reduce_kernel, dim3(nblk(r.T * 4, 64)), dim3(256), 0, st, r, rpartial, nb);
  return hipGetLastError();
}

hipError_t launch_pack_batch(bool bf16, const PackBatchArgs& b, hipStream_t st) {
  const int64_t px = pack_grid_x(b);
  if (px == 0) return hipSuccess;
  if (px < 0) return hipErrorInvalidValue;
  const unsigned bx = (unsigned)px;
  if (bf16) hipLaunchKernelGGL(pack_batch_kernel<uint16_t>, dim3(bx, (unsigned)b.njobs), dim3(256), 0, st, b);
  else hipLaunchKernelGGL(pack_batch_kernel<float>, dim3(bx, (unsigned)b.njobs), dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const CastArgs& a, hipStream_t st) {
  int64_t nmax = 0;
  for (int i = 0; i < a.nseg; ++i) nmax = a.seg[i].n > nmax ? a.seg[i].n : nmax;
  if (a.nseg <= 0 || nmax == 0) return hipSuccess;
  const unsigned bx = nblk(nmax, 256) < 256 ? nblk(nmax, 256) : 256u;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(bx, (unsigned)a.nseg), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, int64_t bytes, hipStream_t st) {
  const int64_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(nblk(n, 256)), dim3(256), 0, st, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace lora
