// fp32 GEMM for the fp32 compute dtype: the same contraction, segments,
// regions, LoRA tail and epilogues (gated and ungated) as the bf16 MFMA
// kernel, computed with fp32 FMAs (no reduced-precision operands), 64x64
// tiles, 4x4 outputs per thread, bounds-checked loads so any shape works.
//
// In dual (gate/up) tiles a thread's four tile columns are
// {gate n, gate n+1, up n, up n+1}, so e and g of one element meet in one
// thread for the activation epilogue.
#include "common.hpp"
#include "kernels.hpp"

namespace lora {
namespace {

constexpr int TM = 64, TN = 64, TK = 16, NTH = 256;

__device__ __forceinline__ void colmap32(bool dual, int nl, int64_t tnl, int& cg, int64_t& n) {
  if (dual) {
    const int tx = nl >> 2, q = nl & 3;
    cg = q >> 1;
    n = tnl * 32 + 2 * tx + (q & 1);
  } else {
    cg = 0;
    n = tnl * 64 + nl;
  }
}

__global__ __launch_bounds__(NTH) void gemm_f32_kernel(const GemmArgs args) {
  __shared__ float sA[TK][TM + 1];
  __shared__ float sB[TK][TN + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t tm = blockIdx.x % args.ntile_m;
  const int64_t tn = blockIdx.x / args.ntile_m;
  int reg = 0;
  for (int p = 1; p < args.nreg; ++p)
    if (tn >= args.reg[p].tile0) reg = p;
  const GemmRegion& R = args.reg[reg];
  const int64_t tnl = tn - R.tile0;
  const int64_t m0 = tm * TM;
  const bool dual = args.dual != 0;

  float acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  const int nseg_total = args.nseg + (args.RL > 0 ? 1 : 0);
  for (int s = 0; s < nseg_total; ++s) {
    const bool lora = s >= args.nseg;
    const int64_t K = lora ? args.RL : args.seg[s].K;
    for (int64_t k0 = 0; k0 < K; k0 += TK) {
      for (int e = tid; e < TK * TM; e += NTH) {
        const int kk = e / TM, ml = e % TM;
        const int64_t m = m0 + ml, k = k0 + kk;
        float v = 0.0f;
        if (m < args.M && k < K) {
          v = lora ? static_cast<const float*>(args.AL)[m * args.ldal + k]
                   : static_cast<const float*>(args.seg[s].A)[m * args.seg[s].lda + k];
        }
        sA[kk][ml] = v;
      }
      for (int e = tid; e < TK * TN; e += NTH) {
        const int kk = e / TN, nl = e % TN;
        int cg;
        int64_t n;
        colmap32(dual, nl, tnl, cg, n);
        const int64_t k = k0 + kk;
        float v = 0.0f;
        if (n < R.N && k < K) {
          if (lora) {
            const int64_t vcol = R.vcol0[cg] + n;
            v = static_cast<const float*>(args.BLt)[vcol * args.ldbl + k];
          } else {
            const BSrc& B = args.seg[s].b[reg][cg];
            const float* p = static_cast<const float*>(B.p);
            v = (args.bkind == B_NN) ? p[k * B.ld + n] : p[n * B.ld + k];
          }
        }
        sB[kk][nl] = v;
      }
      __syncthreads();
      for (int kk = 0; kk < TK; ++kk) {
        float a[4], b[4];
        for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
        for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
        for (int i = 0; i < 4; ++i)
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
      __syncthreads();
    }
  }

  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= args.M) continue;
    if (args.epi == EPI_STORE) {
      for (int j = 0; j < 4; ++j) {
        int cg;
        int64_t n;
        colmap32(false, tx * 4 + j, tnl, cg, n);
        if (n < R.N) static_cast<float*>(R.out)[m * R.ldo + n] = acc[i][j];
      }
    } else if (args.epi == EPI_ACT_FWD) {
      for (int j = 0; j < 2; ++j) {
        int cg;
        int64_t n;
        colmap32(true, tx * 4 + j, tnl, cg, n);
        if (n >= R.N) continue;
        const float e = acc[i][j], g = acc[i][j + 2];
        float phi;
        act_fwd<true>(args.act, e, phi);
        const int64_t off = m * args.ld_act + n;
        static_cast<float*>(args.e_out)[off] = e;
        static_cast<float*>(args.g_out)[off] = g;
        static_cast<float*>(args.h_out)[off] = phi * g;
      }
    } else if (args.epi == EPI_ACT1_FWD) {
      for (int j = 0; j < 4; ++j) {
        int cg;
        int64_t n;
        colmap32(false, tx * 4 + j, tnl, cg, n);
        if (n >= R.N) continue;
        const int64_t off = m * args.ld_act + n;
        static_cast<float*>(args.e_out)[off] = acc[i][j];
        static_cast<float*>(args.h_out)[off] = relu2(acc[i][j]);
      }
    } else if (args.epi == EPI_ACT1_BWD) {
      for (int j = 0; j < 4; ++j) {
        int cg;
        int64_t n;
        colmap32(false, tx * 4 + j, tnl, cg, n);
        if (n >= R.N) continue;
        const int64_t off = m * args.ld_act + n;
        const float u = static_cast<const float*>(args.e_in)[off];
        static_cast<float*>(args.h_out)[off] = relu2(u);
        static_cast<float*>(args.dg_out)[off] = acc[i][j] * relu2_grad(u);
      }
    } else {
      for (int j = 0; j < 4; ++j) {
        int cg;
        int64_t n;
        colmap32(false, tx * 4 + j, tnl, cg, n);
        if (n >= R.N) continue;
        const int64_t off = m * args.ld_act + n;
        const float e = static_cast<const float*>(args.e_in)[off];
        const float g = static_cast<const float*>(args.g_in)[off];
        float phi, dphi;
        act_fwd_bwd<true>(args.act, e, phi, dphi);
        const float dh = acc[i][j];
        static_cast<float*>(args.h_out)[off] = phi * g;
        static_cast<float*>(args.dg_out)[off] = dh * phi;
        static_cast<float*>(args.de_out)[off] = dh * g * dphi;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t st) {
  const int64_t nb = a.ntile_m * a.ntile_n;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)nb), dim3(NTH), 0, st, a);
  return hipGetLastError();
}

}  // namespace lora
