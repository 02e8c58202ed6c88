// bf16 GEMM core for gfx950: 256x256x64 block tiles, 4 wavefronts (2 x 2),
// each wavefront a 128x128 sub-tile of v_mfma_f32_32x32x16_bf16 products with
// fp32 accumulation, operands staged through double-buffered LDS.
//
// What it computes (the base projections and the adapter term of the LoRA
// projections, "LoRA Optimizations" section "Custom autograd functions"; the
// products of the unsloth LoRA_MLP / LoRA_QKV / LoRA_W hunks):
//   forward   Z = X W + (s X A) B        (B operand [K, N], N-contiguous: "NN")
//   backward  dX = dZ W^T + (s P) A^T    (B operand [N, K], K-contiguous: "NT")
// The adapter term is one more K-step of the same MFMA loop: [X | sU] [W ; B].
//
// Epilogues run on the accumulators in registers:
//   EPI_STORE    round to bf16, store;
//   EPI_ACT_FWD  (gate/up tiles) e, g -> bf16, h = phi(e) g from the rounded
//                e, g, store e, g, h;
//   EPI_ACT_BWD  dh -> load e, g, recompute h, dg = dh phi(e),
//                de = dh g phi'(e), store dg, de, h.
//
// MFMA roles.  The weight tile is the MFMA "A" source (32 rows = output
// columns n) and the activation tile the "B" source (32 columns = rows m), so
// each lane ends with 4 consecutive output columns of one row: the epilogue
// writes 8-byte vectors and the gated activation finds e and g of the same
// element in the same lane.
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
#include "common.hpp"
#include "kernels.hpp"

namespace lora {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTH = 256;
constexpr int TILE_CHUNKS = 256 * 8;  // 16-byte chunks per 256 x 64 bf16 tile

// XOR swizzle of the 16-byte chunk index inside a 128-byte LDS row.  Rows read
// together by an MFMA fragment load (8 consecutive rows) and rows written
// together by the transposing store (rows 8 apart) land in different banks.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Block -> tile.  Workgroups are dispatched round-robin over the 8 XCDs, so
// block b runs on XCD b % 8.  Re-number blocks so that each XCD receives a
// contiguous run of logical tiles, and walk logical tiles in groups of 8
// m-tiles (n-major inside a group) so the 32 tiles an XCD holds at once share
// 8 activation panels and 4 weight panels in its L2.
__device__ __forceinline__ void tile_coords(int64_t bid, int64_t nb, int64_t ntm, int64_t ntn,
                                            int64_t& tm, int64_t& tn) {
  const int64_t q = nb >> 3, rem = nb & 7, x = bid & 7, j = bid >> 3;
  const int64_t lid = (x < rem) ? x * (q + 1) + j : rem * (q + 1) + (x - rem) * q + j;
  const int64_t G = 8;
  const int64_t per_group = G * ntn;
  const int64_t grp = lid / per_group;
  const int64_t first_m = grp * G;
  const int64_t gsize = (ntm - first_m < G) ? (ntm - first_m) : G;
  const int64_t in_g = lid - grp * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

// Tile-local weight row nl (0..255) -> (column group, output column).
template <bool DUAL>
__device__ __forceinline__ void colmap(int nl, int64_t tnl, int& cg, int64_t& n) {
  if constexpr (DUAL) {
    cg = (nl >> 6) & 1;
    n = tnl * 128 + (int64_t)(nl >> 7) * 64 + (nl & 63);
  } else {
    cg = 0;
    n = tnl * 256 + nl;
  }
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

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

struct Stage {
  u32x4 a[8];
  u32x4 b[8];       // dense rows, or b[i].x = NF4 code dword
  float bs2[8];     // NF4: scaler-block scale per row
  float bmu[8];     // NF4: mean absmax of the row's weight
  int bq8[8];       // NF4: block code per row
};

template <int BKIND, bool NF4, bool DUAL, int EPI>
__global__ __launch_bounds__(NTH, 1) void gemm_bf16_kernel(const GemmArgs args) {
  __shared__ u32x4 sA[2 * TILE_CHUNKS];
  __shared__ u32x4 sB[2 * TILE_CHUNKS];
  __shared__ float s_lut[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  if (NF4 && tid < 16) {
    const float lv[16] = LORA_NF4_LEVELS_INIT;
    s_lut[tid] = lv[tid];
  }

  int64_t tm, tn;
  tile_coords(blockIdx.x, gridDim.x, args.ntile_m, args.ntile_n, tm, tn);
  int reg = 0;
#pragma unroll
  for (int p = 1; p < 3; ++p)
    if (p < args.nreg && tn >= args.reg[p].tile0) reg = p;
  const int64_t tnl = tn - args.reg[reg].tile0;
  const int64_t NR = args.reg[reg].N;
  const int64_t M = args.M;
  const int64_t m0 = tm * BM;

  // Per-thread constant load geometry.
  const int a_c = tid & 7;          // 16-byte chunk in a 64-wide K slice
  const int a_r0 = tid >> 3;        // first of 8 rows (stride 32)
  const int nn_n8 = tid & 31;       // NN: 8-column group
  const int nn_k8 = tid >> 5;       // NN: 8-row group of K

  // Weight-row geometry (clamped to valid memory; clamped rows only feed
  // output columns that are never stored).
  // Row a_r0 + 32 i of a dual tile is in column group (i >> 1) & 1 for every
  // lane (a_r0 < 32), so the group index is a compile-time constant.
  int64_t nt_col[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int cg;
    int64_t n;
    colmap<DUAL>(a_r0 + 32 * i, tnl, cg, n);
    nt_col[i] = n < NR ? n : NR - 1;
  }
  auto nt_cg = [](int i) { return DUAL ? ((i >> 1) & 1) : 0; };
  int nn_cg;
  int64_t nn_col;
  {
    int64_t n;
    colmap<DUAL>(nn_n8 * 8, tnl, nn_cg, n);
    nn_col = n < NR ? n : NR - 8;
  }
  int64_t a_row[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + a_r0 + 32 * i;
    a_row[i] = m < M ? m : M - 1;
  }

  int64_t ktiles = 0;
  for (int s = 0; s < args.nseg; ++s) ktiles += args.seg[s].K / BK;
  const bool has_lora = args.RL > 0;
  const int64_t KT = ktiles + (has_lora ? 1 : 0);

  // --- global -> registers for one K tile ---------------------------------
  auto load_tile = [&](Stage& st, int seg, int64_t k0, bool lora) {
    if (lora) {
      const int nch = args.RL >> 3;
      const char* AL = static_cast<const char*>(args.AL);
      const char* BL = static_cast<const char*>(args.BLt);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        st.a[i] = u32x4{0, 0, 0, 0};
        st.b[i] = u32x4{0, 0, 0, 0};
        if (a_c < nch) {
          st.a[i] = ld16(AL + (a_row[i] * args.ldal + a_c * 8) * 2);
          const int64_t v = args.reg[reg].vcol0[nt_cg(i)] + nt_col[i];
          st.b[i] = ld16(BL + (v * args.ldbl + a_c * 8) * 2);
        }
      }
      return;
    }
    const GemmSeg& S = args.seg[seg];
    const char* A = static_cast<const char*>(S.A);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.a[i] = ld16(A + (a_row[i] * S.lda + k0 + a_c * 8) * 2);
    if constexpr (BKIND == B_NT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const BSrc& B = S.b[reg][nt_cg(i)];
        if constexpr (NF4) {
          const int64_t flat = nt_col[i] * B.wcols + k0 + a_c * 8;
          st.b[i][0] = *reinterpret_cast<const uint32_t*>(B.codes + (flat >> 1));
          st.bq8[i] = B.q8[flat >> 6];
          st.bs2[i] = B.s2[flat >> 14];
          st.bmu[i] = *B.mu;
        } else {
          st.b[i] = ld16(static_cast<const char*>(B.p) + (nt_col[i] * B.ld + k0 + a_c * 8) * 2);
        }
      }
    } else {
      // In dual tiles the lanes of a wavefront read both column groups; pick
      // the source per lane with selects on uniformly loaded descriptors.
      const BSrc& B0 = S.b[reg][0];
      const BSrc& B1 = S.b[reg][DUAL ? 1 : 0];
      const bool g1 = DUAL && nn_cg == 1;
      if constexpr (NF4) {
        const uint8_t* codes = g1 ? B1.codes : B0.codes;
        const int8_t* q8 = g1 ? B1.q8 : B0.q8;
        const float* s2 = g1 ? B1.s2 : B0.s2;
        const float mu = g1 ? *B1.mu : *B0.mu;
        const int64_t wcols = g1 ? B1.wcols : B0.wcols;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t flat = (k0 + nn_k8 * 8 + i) * wcols + nn_col;
          st.b[i][0] = *reinterpret_cast<const uint32_t*>(codes + (flat >> 1));
          st.bq8[i] = q8[flat >> 6];
          st.bs2[i] = s2[flat >> 14];
          st.bmu[i] = mu;
        }
      } else {
        const char* bp = static_cast<const char*>(g1 ? B1.p : B0.p);
        const int64_t ld = g1 ? B1.ld : B0.ld;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          st.b[i] = ld16(bp + ((k0 + nn_k8 * 8 + i) * ld + nn_col) * 2);
      }
    }
  };

  // --- registers -> LDS -----------------------------------------------------
  auto store_tile = [&](Stage& st, int buf, bool lora) {
    u32x4* dA = sA + buf * TILE_CHUNKS;
    u32x4* dB = sB + buf * TILE_CHUNKS;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = a_r0 + 32 * i;
      dA[row * 8 + (a_c ^ swz(row))] = st.a[i];
    }
    if (lora || BKIND == B_NT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = a_r0 + 32 * i;
        u32x4 v = st.b[i];
        if (NF4 && !lora) v = nf4_decode8(st.b[i][0], nf4_absmax((int8_t)st.bq8[i], st.bs2[i], st.bmu[i]), s_lut);
        dB[row * 8 + (a_c ^ swz(row))] = v;
      }
    } else {
      u32x4 rows[8], cols[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (NF4) rows[i] = nf4_decode8(st.b[i][0], nf4_absmax((int8_t)st.bq8[i], st.bs2[i], st.bmu[i]), s_lut);
        else rows[i] = st.b[i];
      }
      transpose8x8(rows, cols);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = nn_n8 * 8 + j;
        dB[row * 8 + (nn_k8 ^ swz(row))] = cols[j];
      }
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  auto kstep = [&](const u32x4* tA, const u32x4* tB, int ks) {
    {
      const int c = ks * 2 + (lane >> 5);
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rn = wn * 128 + i * 32 + (lane & 31);
        fa[i] = __builtin_bit_cast(bf16x8, tB[rn * 8 + (c ^ swz(rn))]);
        const int rm = wm * 128 + i * 32 + (lane & 31);
        fb[i] = __builtin_bit_cast(bf16x8, tA[rm * 8 + (c ^ swz(rm))]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  // Every tile runs the same 4 K-steps: the LoRA tile is zero-padded past RL.
  // (One uniform path keeps the accumulators in place in AGPRs; a separate
  // short path for the LoRA tile made the compiler copy them.)
  auto compute = [&](int buf) {
    const u32x4* tA = sA + buf * TILE_CHUNKS;
    const u32x4* tB = sB + buf * TILE_CHUNKS;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kstep(tA, tB, ks);
  };

  // --- main loop: prefetch tile t+1 into registers while tile t computes ---
  Stage st;
  int ld_seg = 0;
  int64_t ld_k0 = 0;
  auto next_pos = [&]() {
    ld_k0 += BK;
    if (ld_seg < args.nseg && ld_k0 >= args.seg[ld_seg].K) {
      ++ld_seg;
      ld_k0 = 0;
    }
  };
  const bool first_lora = ld_seg >= args.nseg;
  load_tile(st, ld_seg, ld_k0, first_lora);
  __syncthreads();  // s_lut ready
  store_tile(st, 0, first_lora);
  next_pos();
  __syncthreads();

  for (int64_t t = 0; t < KT; ++t) {
    const int buf = (int)(t & 1);
    const bool has_next = t + 1 < KT;
    const bool nxt_lora = ld_seg >= args.nseg;
    if (has_next) load_tile(st, ld_seg, ld_k0, nxt_lora);
    compute(buf);
    if (has_next) {
      store_tile(st, buf ^ 1, nxt_lora);
      next_pos();
    }
    __syncthreads();
  }

  // --- epilogue --------------------------------------------------------------
  const int mlane = lane & 31;
  const int nhalf = (lane >> 5) * 4;
  if constexpr (EPI == EPI_STORE) {
    char* out = static_cast<char*>(args.reg[reg].out);
    const int64_t ldo = args.reg[reg].ldo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm * 128 + j * 32 + mlane;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = wn * 128 + i * 32 + 8 * g + nhalf;
          int cg;
          int64_t n;
          colmap<DUAL>(nl, tnl, cg, n);
          if (m < M && n < NR) {
            u32x2 v;
            v[0] = pack_bf2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
            v[1] = pack_bf2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            *reinterpret_cast<u32x2*>(out + (m * ldo + n) * 2) = v;
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_ACT_FWD) {
    static_assert(DUAL, "activation forward needs gate/up tiles");
    char* eo = static_cast<char*>(args.e_out);
    char* go = static_cast<char*>(args.g_out);
    char* ho = static_cast<char*>(args.h_out);
    const int64_t ld = args.ld_act;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm * 128 + j * 32 + mlane;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = wn * 128 + i * 32 + 8 * g + nhalf;
          int cg;
          int64_t n;
          colmap<DUAL>(nl, tnl, cg, n);
          if (m < M && n < NR) {
            u32x2 ev, gv, hv;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              ev[h] = pack_bf2(acc[i][j][4 * g + 2 * h], acc[i][j][4 * g + 2 * h + 1]);
              gv[h] = pack_bf2(acc[i + 2][j][4 * g + 2 * h], acc[i + 2][j][4 * g + 2 * h + 1]);
              float p0, p1;
              act_fwd<false>(args.act, lo_bf(ev[h]), p0);
              act_fwd<false>(args.act, hi_bf(ev[h]), p1);
              hv[h] = pack_bf2(p0 * lo_bf(gv[h]), p1 * hi_bf(gv[h]));
            }
            const int64_t off = (m * ld + n) * 2;
            *reinterpret_cast<u32x2*>(eo + off) = ev;
            *reinterpret_cast<u32x2*>(go + off) = gv;
            *reinterpret_cast<u32x2*>(ho + off) = hv;
          }
        }
      }
    }
  } else {
    const char* ei = static_cast<const char*>(args.e_in);
    const char* gi = static_cast<const char*>(args.g_in);
    char* dgo = static_cast<char*>(args.dg_out);
    char* deo = static_cast<char*>(args.de_out);
    char* ho = static_cast<char*>(args.h_out);
    const int64_t ld = args.ld_act;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm * 128 + j * 32 + mlane;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = wn * 128 + i * 32 + 8 * g + nhalf;
          int cg;
          int64_t n;
          colmap<DUAL>(nl, tnl, cg, n);
          if (m < M && n < NR) {
            const int64_t off = (m * ld + n) * 2;
            const u32x2 ev = *reinterpret_cast<const u32x2*>(ei + off);
            const u32x2 gv = *reinterpret_cast<const u32x2*>(gi + off);
            u32x2 dgv, dev, hv;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float d0 = acc[i][j][4 * g + 2 * h], d1 = acc[i][j][4 * g + 2 * h + 1];
              float e0 = lo_bf(ev[h]), e1 = hi_bf(ev[h]);
              float g0 = lo_bf(gv[h]), g1 = hi_bf(gv[h]);
              float p0, q0, p1, q1;
              act_fwd_bwd<false>(args.act, e0, p0, q0);
              act_fwd_bwd<false>(args.act, e1, p1, q1);
              hv[h] = pack_bf2(p0 * g0, p1 * g1);
              dgv[h] = pack_bf2(d0 * p0, d1 * p1);
              dev[h] = pack_bf2(d0 * g0 * q0, d1 * g1 * q1);
            }
            *reinterpret_cast<u32x2*>(dgo + off) = dgv;
            *reinterpret_cast<u32x2*>(deo + off) = dev;
            *reinterpret_cast<u32x2*>(ho + off) = hv;
          }
        }
      }
    }
  }
}

template <int BKIND, bool NF4, bool DUAL, int EPI>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  const int64_t nb = a.ntile_m * a.ntile_n;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BKIND, NF4, DUAL, EPI>), dim3((unsigned)nb), dim3(NTH), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int64_t gemm_tile_cols(bool bf16, bool dual) {
  if (bf16) return dual ? 128 : 256;
  return dual ? 32 : 64;
}
int64_t gemm_tile_rows(bool bf16) { return bf16 ? 256 : 64; }

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t st) {
  const bool nf4 = a.nf4 != 0;
  if (a.bkind == B_NN) {
    if (a.epi == EPI_ACT_FWD) {
      return nf4 ? launch_t<B_NN, true, true, EPI_ACT_FWD>(a, st)
                 : launch_t<B_NN, false, true, EPI_ACT_FWD>(a, st);
    }
    return nf4 ? launch_t<B_NN, true, false, EPI_STORE>(a, st)
               : launch_t<B_NN, false, false, EPI_STORE>(a, st);
  }
  if (a.epi == EPI_ACT_BWD) {
    return nf4 ? launch_t<B_NT, true, false, EPI_ACT_BWD>(a, st)
               : launch_t<B_NT, false, false, EPI_ACT_BWD>(a, st);
  }
  return nf4 ? launch_t<B_NT, true, false, EPI_STORE>(a, st)
             : launch_t<B_NT, false, false, EPI_STORE>(a, st);
}

}  // namespace lora
