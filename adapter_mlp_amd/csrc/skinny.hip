// Rank-r products of the LoRA projections and the small packing kernels.
//
// rowproj   Out[t, j] = sum_k Z[t, k] Bt[j, k]      (T x R, R <= 64)
//   the adapter inputs U = X A (with Bt = A^T) and the hoisted
//   P = dZ B^T (with Bt = B) of the unsloth backward hunks: every P is formed
//   once and then feeds both the A-gradient and the input gradient.
// colproj   Out[k, j] = sum_t Z[t, k] P[t, j]       (K x R, reduction over T)
//   the adapter gradients dA = s X^T P and dB = s U^T dZ (stored transposed).
//
// Both stream one large operand (Z) once from HBM.  The bf16 versions feed
// v_mfma_f32_16x16x32_bf16 straight from 16-byte global loads (rowproj) or
// through a transposing LDS stage (colproj, whose contraction runs down the
// columns of Z).  Reductions are deterministic: fixed wave order in LDS for
// rowproj, per-chunk partials summed in ascending chunk order for colproj.
#include "common.hpp"
#include "kernels.hpp"

namespace lora {
namespace {

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// ---------------------------------------------------------------------------
// rowproj, bf16: one block = 16 rows of Z, 4 wavefronts splitting K in
// interleaved 32-wide steps.  Lane l holds row (l & 15), K group (l >> 4).
// ---------------------------------------------------------------------------
template <int NJ>
__global__ __launch_bounds__(256) void rowproj_bf16_kernel(const RowProjArgs a) {
  __shared__ float red[4][16][NJ * 16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int64_t row = t0 + (lane & 15) < a.T ? t0 + (lane & 15) : a.T - 1;
  const int kg = lane >> 4;
  const char* Z = static_cast<const char*>(a.Z) + (row * a.ldz + kg * 8) * 2;
  const char* Bt = static_cast<const char*>(a.Bt);
  const int64_t nsteps = a.K >> 5;

  f32x4 acc[NJ];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) acc[jb] = f32x4{0, 0, 0, 0};
  const char* bptr[NJ];
  bool bval[NJ];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const int j = jb * 16 + (lane & 15);
    bval[jb] = j < a.R;
    bptr[jb] = Bt + ((int64_t)(bval[jb] ? j : 0) * a.ldb + kg * 8) * 2;
  }
#pragma unroll 4
  for (int64_t ks = w; ks < nsteps; ks += 4) {
    const u32x4 zv = ld16(Z + ks * 64);
    const bf16x8 za = __builtin_bit_cast(bf16x8, zv);
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
      u32x4 bv = ld16(bptr[jb] + ks * 64);
      if (!bval[jb]) bv = u32x4{0, 0, 0, 0};
      acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za, __builtin_bit_cast(bf16x8, bv), acc[jb], 0, 0, 0);
    }
  }
  // acc[jb][v] = Out[t0 + 4 (lane >> 4) + v, 16 jb + (lane & 15)] (this wave's K share)
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[w][4 * (lane >> 4) + v][jb * 16 + (lane & 15)] = acc[jb][v];
  __syncthreads();
  const int R2 = a.R2 > a.R ? a.R2 : a.R;
  for (int e = tid; e < 16 * R2; e += 256) {
    const int rl = e / R2, j = e % R2;
    const int64_t t = t0 + rl;
    if (t >= a.T) continue;
    float v = 0.0f;
    if (j < a.R) v = ((red[0][rl][j] + red[1][rl][j]) + red[2][rl][j]) + red[3][rl][j];
    if (a.out1 && j < a.R)
      static_cast<uint16_t*>(a.out1)[t * a.ld1 + a.off1 + j] = (uint16_t)f2bf(v);
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
// colproj, bf16.  Block = 64 columns of Z (k) x one chunk of T.  Per 256-row
// step: Z [256 x 64] and P [256 x R] are loaded as 8x8 sub-blocks, transposed
// in registers and stored T-contiguous in LDS (Zt [64][256], Pt [R][256]);
// then wave w multiplies Zt rows 16w..16w+15 by Pt over the 256 rows.
// LDS rows are 32 chunks of 16 bytes, chunk index XOR-swizzled by the row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void transpose8x8(const u32x4 (&r)[8], u32x4 (&o)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = r[2 * q][p], hi = r[2 * q + 1][p];
      o[2 * p][q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      o[2 * p + 1][q] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
    }
}

template <int NJ>
__global__ __launch_bounds__(256) void colproj_bf16_kernel(const ColProjArgs a, int64_t rows_per_chunk) {
  __shared__ u32x4 Zt[64 * 32];
  __shared__ u32x4 Pt[NJ * 16 * 32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t k0 = (int64_t)blockIdx.x * 64;
  const int64_t c = blockIdx.y;
  const int64_t tbeg = c * rows_per_chunk;
  int64_t tend = tbeg + rows_per_chunk;
  if (tend > a.T) tend = a.T;
  const char* Z = static_cast<const char*>(a.Z);
  const char* P = static_cast<const char*>(a.P);
  const int kc = tid & 7, tg = tid >> 3;   // Z: 8-column chunk, 8-row group
  const int npair = (a.R >> 3) * 32;       // P: (8-column chunk, 8-row group) pairs
  const int pjc = tid >> 5, ptg = tid & 31;

  f32x4 acc[NJ];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) acc[jb] = f32x4{0, 0, 0, 0};

  for (int64_t ts = tbeg; ts < tend; ts += 256) {
    {
      u32x4 r[8], o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t t = ts + tg * 8 + i;
        r[i] = t < tend ? ld16(Z + (t * a.ldz + k0 + kc * 8) * 2) : u32x4{0, 0, 0, 0};
      }
      transpose8x8(r, o);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = kc * 8 + j;
        Zt[row * 32 + (tg ^ (row & 31))] = o[j];
      }
    }
    if (tid < npair) {
      u32x4 r[8], o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t t = ts + ptg * 8 + i;
        r[i] = t < tend ? ld16(P + (t * a.ldp + pjc * 8) * 2) : u32x4{0, 0, 0, 0};
      }
      transpose8x8(r, o);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = pjc * 8 + j;
        Pt[row * 32 + (ptg ^ (row & 31))] = o[j];
      }
    }
    // rows of Pt past R hold stale data only for j >= R, which is never stored
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int ch = s * 4 + (lane >> 4);
      const int zr = w * 16 + (lane & 15);
      const bf16x8 za = __builtin_bit_cast(bf16x8, Zt[zr * 32 + (ch ^ (zr & 31))]);
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        const int pr = jb * 16 + (lane & 15);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, Pt[pr * 32 + (ch ^ (pr & 31))]);
        acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za, pb, acc[jb], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // acc[jb][v] = Out[k0 + 16 w + 4 (lane >> 4) + v, 16 jb + (lane & 15)]
  const int Rp = NJ * 16;
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t k = k0 + w * 16 + 4 * (lane >> 4) + v;
      a.partial[(c * a.K + k) * Rp + jb * 16 + (lane & 15)] = acc[jb][v];
    }
}

__device__ __forceinline__ void colproj_store(const ColProjArgs& a, bool bf16, int64_t k, int j, float v) {
  const int q = j / a.seg_w, jj = j % a.seg_w;
  const float o = a.scales[q] * v;
  const int64_t idx = a.transposed ? (int64_t)jj * a.K + k : k * a.seg_w + jj;
  if (bf16) static_cast<uint16_t*>(a.dest[q])[idx] = (uint16_t)f2bf(o);
  else static_cast<float*>(a.dest[q])[idx] = o;
}

__global__ void colproj_reduce_kernel(const ColProjArgs a, int Rp) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.K * a.R) return;
  const int64_t k = e / a.R;
  const int j = (int)(e % a.R);
  float v = 0.0f;
  for (int c = 0; c < a.nchunk; ++c) v += a.partial[(c * a.K + k) * Rp + j];
  colproj_store(a, true, k, j, v);
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
template <typename E>
__global__ void pack_lora_b_kernel(const PackLoraArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.vcols * a.RL) return;
  const int64_t v = e / a.RL;
  const int kk = (int)(e % a.RL);
  E val = E(0);
  for (int p = 0; p < a.nparts; ++p) {
    const PackPart& q = a.part[p];
    if (v >= q.v0 && v < q.v0 + q.nv && kk >= q.k0 && kk < q.k0 + q.w) {
      const int64_t n = v - q.v0, i = kk - q.k0;
      const E* src = static_cast<const E*>(q.src);
      val = q.nn ? src[i * q.ld + n] : src[n * q.ld + i];
    }
  }
  const int64_t o = a.kmajor ? (int64_t)kk * a.vcols + v : e;
  static_cast<E*>(a.out)[o] = val;
}

struct CatSrcs {
  const void* s[4];
};

template <typename E>
__global__ void pack_cat_t_kernel(E* out, int64_t K, int Rpad, int w, int nparts, CatSrcs srcs) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)Rpad * K) return;
  const int j = (int)(e / K);
  const int64_t k = e % K;
  E val = E(0);
  if (j < nparts * w) val = static_cast<const E*>(srcs.s[j / w])[k * w + (j % w)];
  out[e] = val;
}

__global__ void zero_kernel(uint32_t* p, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) p[e] = 0u;
}

inline unsigned nblk(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }

}  // namespace

int colproj_nchunk(int64_t T, int64_t K) {
  const int64_t steps = (T + 255) / 256;
  if (steps == 0) return 0;
  const int64_t kblocks = K / 64;
  int64_t want = (2048 + kblocks - 1) / kblocks;
  if (want < 1) want = 1;
  return (int)(want < steps ? want : steps);
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
  const dim3 grid(nblk(a.T, 16));
  switch ((a.R + 15) / 16) {
    case 1: hipLaunchKernelGGL(rowproj_bf16_kernel<1>, grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(rowproj_bf16_kernel<2>, grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL(rowproj_bf16_kernel<3>, grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL(rowproj_bf16_kernel<4>, grid, dim3(256), 0, st, a); break;
  }
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
    const int64_t steps = (a.T + 255) / 256;
    const int64_t steps_per_chunk = (steps + a.nchunk - 1) / a.nchunk;
    const int64_t rows_per_chunk = steps_per_chunk * 256;
    a.nchunk = (int)((a.T + rows_per_chunk - 1) / rows_per_chunk);
    const dim3 grid((unsigned)(a.K / 64), (unsigned)a.nchunk);
    switch (NJ) {
      case 1: hipLaunchKernelGGL(colproj_bf16_kernel<1>, grid, dim3(256), 0, st, a, rows_per_chunk); break;
      case 2: hipLaunchKernelGGL(colproj_bf16_kernel<2>, grid, dim3(256), 0, st, a, rows_per_chunk); break;
      case 3: hipLaunchKernelGGL(colproj_bf16_kernel<3>, grid, dim3(256), 0, st, a, rows_per_chunk); break;
      default: hipLaunchKernelGGL(colproj_bf16_kernel<4>, grid, dim3(256), 0, st, a, rows_per_chunk); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(colproj_reduce_kernel, dim3(nblk(a.K * a.R, 256)), dim3(256), 0, st, a, NJ * 16);
  return hipGetLastError();
}

hipError_t launch_pack_lora_b(bool bf16, const PackLoraArgs& a, hipStream_t st) {
  const int64_t n = a.vcols * a.RL;
  if (n == 0) return hipSuccess;
  if (bf16) hipLaunchKernelGGL(pack_lora_b_kernel<uint16_t>, dim3(nblk(n, 256)), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(pack_lora_b_kernel<float>, dim3(nblk(n, 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pack_cat_t(bool bf16, void* out, int64_t K, int Rpad, int w, int nparts,
                             const void* const* srcs, hipStream_t st) {
  CatSrcs s{};
  for (int i = 0; i < nparts && i < 4; ++i) s.s[i] = srcs[i];
  const int64_t n = (int64_t)Rpad * K;
  if (n == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(pack_cat_t_kernel<uint16_t>, dim3(nblk(n, 256)), dim3(256), 0, st,
                       static_cast<uint16_t*>(out), K, Rpad, w, nparts, s);
  else
    hipLaunchKernelGGL(pack_cat_t_kernel<float>, dim3(nblk(n, 256)), dim3(256), 0, st,
                       static_cast<float*>(out), K, Rpad, w, nparts, s);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, int64_t bytes, hipStream_t st) {
  const int64_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(nblk(n, 256)), dim3(256), 0, st, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace lora
