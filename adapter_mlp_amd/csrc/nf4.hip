// NF4 storage of frozen base weights: quantize, dequantize, unpack
// ("loralei" README, section "Use", QLoRA paragraphs: NF4 codes in blocks of
// 64, block scales double-quantized in scaler blocks of 256, numel divisible
// by 64 * 256).  The format details the page leaves open are fixed as:
//   a_b  = max |w| over the 64-element block b
//   code = nearest NF4 level to fl32(w / a_b), ties to the lower level;
//          a_b = 0 gives the zero level
//   mu   = fl32(S / nblocks), S the fp64 sum of all a_b, each scaler block
//          summed in ascending order, then the scaler-block sums in order
//   d_b  = fl32(a_b - mu); s2 = fl32(max_S |d_b| / 127);
//   q8_b = clamp(rint(fl32(d_b / s2)), -127, 127)  (0 when s2 = 0)
//   dequant: a' = fl32(fl32(q8_b s2) + mu), w' = fl32(c[code] a')
// All steps use explicitly rounded fp32 / fp64 operations so the results are
// bit-for-bit reproducible.
#include "common.hpp"
#include "kernels.hpp"

namespace lora {

const float kNF4Levels[16] = LORA_NF4_LEVELS_INIT;

namespace {

__constant__ float c_levels[16] = LORA_NF4_LEVELS_INIT;

__device__ __forceinline__ float load_w(const void* W, bool bf16, int64_t i) {
  return bf16 ? bf2f(static_cast<const uint16_t*>(W)[i]) : static_cast<const float*>(W)[i];
}

// One thread per 64-element block: absmax and the 64 codes.
__global__ void nf4_codes_kernel(const void* W, bool bf16, int64_t nblocks, uint8_t* codes, float* absmax) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = c_levels[threadIdx.x];
  __syncthreads();
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const int64_t base = b * NF4_BLOCK;
  float a = 0.0f;
  for (int i = 0; i < NF4_BLOCK; ++i) a = fmaxf(a, fabsf(load_w(W, bf16, base + i)));
  absmax[b] = a;
  uint32_t packed[8];
  for (int q = 0; q < 8; ++q) {
    uint32_t word = 0;
    for (int e = 0; e < 8; ++e) {
      const float w = load_w(W, bf16, base + q * 8 + e);
      const float x = a > 0.0f ? __fdiv_rn(w, a) : 0.0f;
      int best = 0;
      float bd = fabsf(__fsub_rn(x, lv[0]));
      for (int i = 1; i < 16; ++i) {
        const float d = fabsf(__fsub_rn(x, lv[i]));
        if (d < bd) {
          bd = d;
          best = i;
        }
      }
      // element 2p goes to the high nibble of byte p
      const int byte = e >> 1;
      const int shift = 8 * byte + ((e & 1) ? 0 : 4);
      word |= (uint32_t)best << shift;
    }
    packed[q] = word;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(codes + b * (NF4_BLOCK / 2));
  dst[0] = u32x4{packed[0], packed[1], packed[2], packed[3]};
  dst[1] = u32x4{packed[4], packed[5], packed[6], packed[7]};
}

// One thread per scaler block: fp64 sum of its 256 absmaxes, ascending.
__global__ void nf4_partial_sum_kernel(const float* absmax, int64_t nsb, double* part) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= nsb) return;
  double acc = 0.0;
  for (int i = 0; i < NF4_SCALER; ++i) acc = __dadd_rn(acc, (double)absmax[s * NF4_SCALER + i]);
  part[s] = acc;
}

// Single thread: scaler-block sums in ascending order, then the mean.
__global__ void nf4_mean_kernel(const double* part, int64_t nsb, int64_t nblocks, float* mu) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double acc = 0.0;
  for (int64_t s = 0; s < nsb; ++s) acc = __dadd_rn(acc, part[s]);
  *mu = (float)__ddiv_rn(acc, (double)nblocks);
}

// One 64-lane wavefront per scaler block (4 blocks per lane).
__global__ __launch_bounds__(64) void nf4_double_quant_kernel(const float* absmax, const float* mu_p,
                                                              int8_t* q8, float* s2) {
  const int64_t s = blockIdx.x;
  const int lane = threadIdx.x;
  const float mu = *mu_p;
  float d[4];
  float m = 0.0f;
  for (int i = 0; i < 4; ++i) {
    d[i] = __fsub_rn(absmax[s * NF4_SCALER + lane * 4 + i], mu);
    m = fmaxf(m, fabsf(d[i]));
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const float sc = __fdiv_rn(m, 127.0f);
  if (lane == 0) s2[s] = sc;
  for (int i = 0; i < 4; ++i) {
    int q = 0;
    if (sc > 0.0f) {
      float r = rintf(__fdiv_rn(d[i], sc));
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      q = (int)r;
    }
    q8[s * NF4_SCALER + lane * 4 + i] = (int8_t)q;
  }
}

// One thread per 8 elements.
__global__ void nf4_dequant_kernel(const uint8_t* codes, const int8_t* q8, const float* s2, const float* mu_p,
                                   int64_t ngroups, void* out, bool bf16) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= ngroups) return;
  const int64_t flat = g * 8;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + flat / 2);
  const float a = nf4_absmax(q8[flat / NF4_BLOCK], s2[flat / NF4_GROUP], *mu_p);
  float v[8];
  for (int q = 0; q < 4; ++q) {
    const uint32_t byte = (w >> (8 * q)) & 0xffu;
    v[2 * q] = __fmul_rn(c_levels[byte >> 4], a);
    v[2 * q + 1] = __fmul_rn(c_levels[byte & 0xfu], a);
  }
  if (bf16) {
    u32x4 o;
    for (int q = 0; q < 4; ++q) o[q] = f2bf(v[2 * q]) | (f2bf(v[2 * q + 1]) << 16);
    reinterpret_cast<u32x4*>(out)[g] = o;
  } else {
    f32x4* o = reinterpret_cast<f32x4*>(out) + 2 * g;
    o[0] = f32x4{v[0], v[1], v[2], v[3]};
    o[1] = f32x4{v[4], v[5], v[6], v[7]};
  }
}

__global__ void nf4_unpack_kernel(const uint8_t* codes, int64_t ngroups, uint8_t* out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= ngroups) return;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + g * 4);
  uint32_t lo = 0, hi = 0;
  for (int q = 0; q < 2; ++q) {
    const uint32_t byte = (w >> (8 * q)) & 0xffu;
    lo |= ((byte >> 4) << (16 * q)) | ((byte & 0xfu) << (16 * q + 8));
  }
  for (int q = 0; q < 2; ++q) {
    const uint32_t byte = (w >> (8 * (q + 2))) & 0xffu;
    hi |= ((byte >> 4) << (16 * q)) | ((byte & 0xfu) << (16 * q + 8));
  }
  reinterpret_cast<u32x2*>(out)[g] = u32x2{lo, hi};
}

inline unsigned nblk(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }

}  // namespace

size_t nf4_quantize_ws_bytes(int64_t numel) {
  const int64_t nblocks = numel / NF4_BLOCK, nsb = numel / NF4_GROUP;
  return (size_t)(((nblocks * 4 + 255) / 256) * 256 + nsb * 8);
}

hipError_t launch_nf4_quantize(const void* W, int64_t numel, bool bf16, uint8_t* codes, int8_t* q8,
                               float* s2, float* mu, void* ws, hipStream_t st) {
  const int64_t nblocks = numel / NF4_BLOCK, nsb = numel / NF4_GROUP;
  float* absmax = static_cast<float*>(ws);
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) + ((nblocks * 4 + 255) / 256) * 256);
  hipLaunchKernelGGL(nf4_codes_kernel, dim3(nblk(nblocks, 256)), dim3(256), 0, st, W, bf16, nblocks, codes, absmax);
  hipLaunchKernelGGL(nf4_partial_sum_kernel, dim3(nblk(nsb, 64)), dim3(64), 0, st, absmax, nsb, part);
  hipLaunchKernelGGL(nf4_mean_kernel, dim3(1), dim3(64), 0, st, part, nsb, nblocks, mu);
  hipLaunchKernelGGL(nf4_double_quant_kernel, dim3((unsigned)nsb), dim3(64), 0, st, absmax, mu, q8, s2);
  return hipGetLastError();
}

hipError_t launch_nf4_dequant(const uint8_t* codes, const int8_t* q8, const float* s2, const float* mu,
                              int64_t numel, void* out, bool bf16, hipStream_t st) {
  const int64_t ng = numel / 8;
  hipLaunchKernelGGL(nf4_dequant_kernel, dim3(nblk(ng, 256)), dim3(256), 0, st, codes, q8, s2, mu, ng, out, bf16);
  return hipGetLastError();
}

hipError_t launch_nf4_unpack(const uint8_t* codes, int64_t numel, uint8_t* out, hipStream_t st) {
  const int64_t ng = numel / 8;
  hipLaunchKernelGGL(nf4_unpack_kernel, dim3(nblk(ng, 256)), dim3(256), 0, st, codes, ng, out);
  return hipGetLastError();
}

}  // namespace lora
