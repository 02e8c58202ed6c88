// bf16 GEMM core for gfx950: 256x256x64 block tiles, 8 wavefronts in two
// groups that alternate between MFMA clusters and LDS fragment reads,
// v_mfma_f32_16x16x32_bf16 (dense weights) or v_mfma_f32_32x32x16_bf16 (NF4
// weights) with fp32 accumulation, operands moved from global memory into LDS
// without passing through registers.
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
//                de = dh g phi'(e), store dg, de, h;
//   EPI_ACT1_FWD (ungated ReLU^2 MLP) u -> bf16, h = relu(u)^2 from the
//                rounded u, store u, h;
//   EPI_ACT1_BWD dh -> load u, recompute h, du = dh 2 relu(u), store du, h.
// Each wavefront stages its results through a private LDS region so global
// loads and stores move whole 16-byte chunks of consecutive columns.
//
// MFMA roles.  The weight tile is the MFMA "A" source (rows = output columns
// n) and the activation tile the "B" source (columns = rows m), so each lane
// ends with 4 consecutive output columns of one row, and the gated activation
// finds e and g of the same element in the same lane.
//
// MFMA shape.  Under a sustained MFMA load the chip is power-limited, and the
// 16x16x32 instruction, which accumulates over twice the K of 32x32x16 and so
// reads and writes half the accumulator bytes per flop, holds a higher clock:
// in a loop of nothing but MFMAs on one block per CU (same operand and
// accumulator registers) 1.98 against 1.74 GHz.  The dense kernels therefore
// use 16x16x32 blocks.  The NF4 kernels keep 32x32x16: their unpack is
// interleaved with the MFMA cluster at about five vector instructions per
// MFMA, and their matrix cores are busy less than half the time, so the power
// limit binds less.
//
// Operands are read with buffer loads: rows past the end of a matrix read as
// zero, which covers ragged M and N tiles without clamping.
//
// NF4 base weights (QLoRA) are unpacked inside the same loop.  Per 64-element
// block, the absmax is rebuilt from its int8 code, its scaler block's fp32
// scale and the global mean; the 16 products fl32(level * absmax) are rounded
// to bf16 once into a register table, and every 4-bit code is looked up in it
// with byte permutes.  The bf16 tile then goes to LDS in the dense layout
// ("loralei" README, section "Use": unpack and double-scale reconstruction
// fused into the matmul).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace lora {

// Per-block timing (a separate build, -DLORA_BLOCK_TIMING, read by
// lora_block_times): wavefront 0 of every block records the 100 MHz real-time
// clock at kernel entry, at the start and the end of its K loop and after the
// epilogue, the shader clock (s_memtime) at entry and exit, its hardware ids
// and the launch shape, in the slot of its kernel family ((NF4 ? 4 : 0) +
// activation forward 0, activation backward 1, NT store 2, NN store 3).  A
// family's slots hold its latest launch.  The normal build compiles none of it.
// The stamps are held in scalar registers until the exit: the dense kernels
// compile without spills, the NF4 kernels spill 2 to 5 scalar and up to 6
// vector registers, so their timing-build figures run slower than the normal
// build (storing each stamp when taken, or holding 32-bit stamps, spilled more).
#ifdef LORA_BLOCK_TIMING
constexpr bool kBlockTiming = true;
constexpr int kTimedBlocks = 8192;
__device__ unsigned long long block_times[8][kTimedBlocks][8];
#else
constexpr bool kBlockTiming = false;
#endif
// Per-phase timing (another build, -DLORA_PHASE_TIMING, read by
// lora_phase_times): in blocks 0..63, lane 0 of wavefronts 0 and 4 (the first
// of each group) reads the shader clock at every phase boundary of K step
// kPhaseStep and at the start of the next step, and stores them with the K
// step count after the loop, in the slot of the kernel family (as
// block_times).  Group 0 records: MFMA cluster start, its end, after the wait
// for its loads, read phase start (after the barrier), read phase end; group
// 1: read phase start, its end, MFMA cluster start (after the barrier), its
// end.  The stamps are held in scalar registers through the loop, which
// changes the register allocation of this build.
#ifdef LORA_PHASE_TIMING
constexpr int kPhaseStep = 21;
__device__ unsigned long long phase_times[8][64][2][8];
#endif

namespace {

constexpr int BM = 256, BK = 64;

// XOR swizzle of the 16-byte chunk index inside a 128-byte LDS row (K-contiguous
// tiles).  A 16-byte LDS read is served a group of lanes at a time, and lanes
// of one group that touch the same bank are serialised.  Timed on the device
// (8 wavefronts of back-to-back ds_read_b128, in-bounds offsets):
//   32x32x16 fragments (lane l: row l % 32, chunk 2 ks + l / 32), swizzle
//     (r ^ r >> 3) & 7: full rate, the same as 64 consecutive 16-byte chunks;
//   16x16x32 fragments (lane l: row l % 16, chunk 4 ks + l / 16): half rate
//     under (r ^ r >> 3) & 7 and several other swizzles, full rate under r & 7.
// The dense kernels (16x16x32 reads) therefore take r & 7, and the NF4
// kernels (32x32x16 reads, and an unpack that writes 64 consecutive rows at
// one chunk) keep (r ^ r >> 3) & 7.
template <bool M16>
__device__ __forceinline__ int swz(int row) {
  return M16 ? (row & 7) : ((row ^ (row >> 3)) & 7);
}

// NN weight tiles (256-byte rows of 16 chunks): chunk c of K row k sits at
// c ^ nn_swz(k).  A dense tile is written by global -> LDS loads that fill
// whole rows, so only the transposing fragment reads (4 rows x 4 chunks at a
// time) need spreading over the banks: 4 (k & 3).  Under the 16x16x32 reads
// (lanes 16 g + 4 j + q: K row 8 g + j) the bank-conflict counter charges each
// transposing read two extra cycles, which 4 (k & 3) ^ 2 (k >> 3 & 1) removes;
// that layout measured no faster (those reads issue at about one per five
// cycles and wavefront anyway, and it needs two more offset registers), so the
// plain one stays.
// An NF4 tile is written by the unpack, 16 lanes at a time over 8 rows and 2
// chunks 8 apart, so its swizzle also spreads 8 consecutive rows:
// 4 (k & 3) + ((k >> 1) & 3) keeps any 4 aligned rows x 4 aligned chunks and
// any 8 aligned rows x {c, c + 8} on distinct chunk positions.
template <bool NF4>
__device__ __forceinline__ int nn_swz(int k) {
  return NF4 ? (((k & 3) << 2) | ((k >> 1) & 3)) : ((k & 3) << 2);
}

// v_permlane32_swap_b32: lo = (a in lanes 0-31, b of lanes 0-31 in lanes
// 32-63), hi = (a of lanes 32-63 in lanes 0-31, b in lanes 32-63).  The
// operands pass through empty asm statements: applied directly to elements
// of an MFMA accumulator tuple, the swap was compiled with both operands
// taken from one register.
__device__ __forceinline__ void swap_lane_halves(float a, float b, float& lo, float& hi) {
  uint32_t x = __builtin_bit_cast(uint32_t, a), y = __builtin_bit_cast(uint32_t, b);
  asm volatile("" : "+v"(x), "+v"(y));
  const auto s = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  uint32_t p = s[0], q = s[1];
  asm volatile("" : "+v"(p), "+v"(q));
  lo = __builtin_bit_cast(float, p);
  hi = __builtin_bit_cast(float, q);
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
// contiguous run of logical tiles, and walk logical tiles in groups of G
// m-tiles (n-major inside a group): the 32 tiles an XCD holds at once then
// share G activation panels and 32 / G weight panels in its L2 (8 x 4 or
// 4 x 8 panels fetch the same bytes; measured, groups of 4 suit the
// activation-epilogue GEMMs and groups of 8 the store GEMMs, the defaults; a
// call's plan may choose another G).  All arguments are uniform.
__device__ __forceinline__ void tile_coords(int bid, int nb, int ntm, int ntn, int G, int& tm, int& tn) {
  const int q = nb >> 3, rem = nb & 7, x = bid & 7, j = bid >> 3;
  const int lid = (x < rem) ? x * (q + 1) + j : rem * (q + 1) + (x - rem) * q + j;
  const int per_group = G * ntn;
  const int grp = lid / per_group;
  const int first_m = grp * G;
  const int gsize = (ntm - first_m < G) ? (ntm - first_m) : G;
  const int in_g = lid - grp * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
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

// A wavefront's accumulators (its 64 output columns x 128 rows) as 32x32 MFMA
// blocks, f32x16 [2][4] (block i: columns 32 i.., block j: rows 32 j..; lane l
// holds row 32 j + l % 32, columns 32 i + 8 g + 4 (l / 32) + v in registers
// 4 g + v), or as 16x16 blocks, f32x4 [4][8] (block i: columns 16 i.., block
// j: rows 16 j..; lane l holds row 16 j + l % 16, columns 16 i + 4 (l / 16) + v).
// The epilogues read either as quads: quad q (0..7) of 32-row pass j is four
// consecutive columns qcol .. qcol + 3 of row qrow of the pass, in one lane.
// In gate/up tiles quads q < 4 hold gate columns and quad q + 4 the up columns
// of the same outputs.
__device__ __forceinline__ f32x4 quad(const f32x16 (&acc)[2][4], int q, int j) {
  const int i = q >> 2, g = q & 3;
  return f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
}
__device__ __forceinline__ int qcol(const f32x16 (&)[2][4], int q, int lane) {
  return 32 * (q >> 2) + 8 * (q & 3) + 4 * (lane >> 5);
}
__device__ __forceinline__ int qrow(const f32x16 (&)[2][4], int, int lane) { return lane & 31; }
__device__ __forceinline__ f32x4 quad(const f32x4 (&acc)[4][8], int q, int j) { return acc[q >> 1][2 * j + (q & 1)]; }
__device__ __forceinline__ int qcol(const f32x4 (&)[4][8], int q, int lane) { return 16 * (q >> 1) + 4 * (lane >> 4); }
__device__ __forceinline__ int qrow(const f32x4 (&)[4][8], int q, int lane) { return 16 * (q & 1) + (lane & 15); }

// Epilogue: each wavefront stages its results (WN output tile columns x 128
// rows, read from the accumulators as quads, one 32-row pass at a time)
// through a private LDS region -- the operand buffers are free once the K
// loop has ended -- so global loads and stores move 16-byte chunks of
// consecutive columns.
// Backward activation epilogues: region 0 holds the fp32 dh rows of a pass,
// then (once read) the bf16 gradient rows [NP][32][WN + 8] of the fused
// rank-r products; then h rows [32][WN + 8] bf16, Pd rows [32][16] bf16 and
// U rows [NP][32][16] bf16.
template <int WN, int EPI>
constexpr int bwd_region0() {
  return 32 * (WN + 4) * 4 > (EPI == EPI_ACT_BWD ? 2 : 1) * 32 * (WN + 8) * 2
             ? 32 * (WN + 4) * 4
             : (EPI == EPI_ACT_BWD ? 2 : 1) * 32 * (WN + 8) * 2;
}
// Staging bytes one wavefront needs for a WN-column epilogue.
template <int WN, int EPI>
constexpr int epi_stage_bytes() {
  return EPI == EPI_STORE      ? 32 * (WN + 4) * 4
         : EPI == EPI_ACT_FWD  ? (3 * 32 * (WN / 2 + 8) * 2 > 8 * 64 * 16 ? 3 * 32 * (WN / 2 + 8) * 2 : 8 * 64 * 16)
         : EPI == EPI_ACT1_FWD ? 2 * 32 * (WN + 8) * 2
                               : bwd_region0<WN, EPI>() + 32 * (WN + 8) * 2 + 32 * 16 * 2 +
                                     (EPI == EPI_ACT_BWD ? 2 : 1) * 32 * 16 * 2;
}

// U = h Ad formed by a forward activation epilogue (u_part set): HC h columns
// per wavefront (32 in gate/up tiles, 64 in ReLU^2 tiles), K blocks of 32.
// Per 32-row pass, the staged h rows (row-major, pitch LD) feed 16x16x32
// MFMAs: M = 16 rows, N = the 16 adapter columns, K = 32 h columns; lane l
// holds the Ad^T fragment of adapter column l % 16, h columns 8 (l / 16) ..
// + 7 of each K block (zero past u_R and NR).  At the end the four
// wavefronts of a row group (same rows) are added in fixed order in LDS and
// wavefront wn writes the sums of pass wn into the tile's slice of u_part.
template <int HC>
struct FusedU {
  static constexpr int KB = HC / 32;
  bf16x8 adf[KB];
  f32x4 acc[4][2];
  __device__ __forceinline__ void init(const GemmArgs& args, int64_t nbase, int64_t NR, int lane) {
    // zero sums for a wavefront whose columns lie past NR (it runs no pass)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) acc[jj][mb] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      adf[kb] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
      const int jr = lane & 15;
      const int64_t n = nbase + 32 * kb + 8 * (lane >> 4);
      if (jr < args.u_R && n < NR)
        adf[kb] = *reinterpret_cast<const bf16x8*>(static_cast<const char*>(args.ad_t) + (jr * args.ld_adt + n) * 2);
    }
  }
  template <int J, int LD>
  __device__ __forceinline__ void pass(const uint16_t* hstage, int lane) {
    const lds_char* hs = (const lds_char*)hstage;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x4 a = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 hf = __builtin_bit_cast(
            bf16x8, lds_read16(hs + ((mb * 16 + (lane & 15)) * LD + 32 * kb + 8 * (lane >> 4)) * 2));
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hf, adf[kb], a, 0, 0, 0);
      }
      acc[J][mb] = a;
    }
  }
  // wstage: this wavefront's staging (EB bytes per wavefront, wavefront wn of its group)
  template <int EB>
  __device__ __forceinline__ void finish(const GemmArgs& args, char* wstage, int64_t mw, int64_t tnb, int64_t M,
                                         int wn, int lane) {
    f32x4* red = reinterpret_cast<f32x4*>(wstage);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) red[(jj * 2 + mb) * 64 + lane] = acc[jj][mb];
    __syncthreads();
    const char* g0 = wstage - wn * EB;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x4 sum = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int q = 0; q < 4; ++q) sum += reinterpret_cast<const f32x4*>(g0 + q * EB)[(wn * 2 + mb) * 64 + lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = mw + 32 * wn + 16 * mb + 4 * (lane >> 4) + v;
        if (m < M) args.u_part[(tnb * M + m) * 16 + (lane & 15)] = sum[v];
      }
    }
  }
};

// Every feature width of a bf16 call is a multiple of 64, so the WN / 2 (gate/up
// tiles) or WN (other tiles) output columns of a wavefront lie wholly inside or
// wholly past the region: the column check is uniform across the wavefront.
// Rows past M are handled by the range-checked buffer accesses (loads read
// zero, stores are dropped), so the epilogues carry no per-lane branch.
template <int WN, bool DUAL, int EPI, int ACT, typename ACC>
__device__ __forceinline__ void run_epilogue_w(const ACC& acc, char* wstage, const GemmArgs& args,
                                               int reg, int64_t mw, int64_t nbase, int64_t NR, int64_t M,
                                               int lane, int wm, int wn, int kp) {
  // kp >= 0: this block computes K part kp of a split tile (fp32 partial sums)
  static_assert(WN == 64, "the quads cover 64 columns per wavefront");
  constexpr int NQ = WN / 8;             // quads per 32-row pass
  const bool cols_ok = nbase < NR;  // uniform
  if constexpr (EPI == EPI_STORE) {
    if (kp >= 0) {
      // split-K part: fp32 sums through a [32][WN] fp32 staging, 16-byte stores
      constexpr int LD = WN + 4;
      constexpr int CPR = WN / 4;          // 4-float chunks per row
      constexpr int RPP = 64 / CPR;
      float* stg = reinterpret_cast<float*>(wstage);
      const brsrc ro = make_rsrc(args.kpart + (int64_t)kp * M * NR, M * NR * 4);
      if (!cols_ok) return;
      for4([&](auto jc) {
        constexpr int j = decltype(jc)::value;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          *reinterpret_cast<f32x4*>(stg + qrow(acc, q, lane) * LD + qcol(acc, q, lane)) = quad(acc, q, j);
        wave_sync();
#pragma unroll
        for (int it = 0; it < 32 / RPP; ++it) {
          const int row = it * RPP + lane / CPR, c4 = lane % CPR;
          const f32x4 v = *reinterpret_cast<const f32x4*>(stg + row * LD + c4 * 4);
          const int64_t m = mw + j * 32 + row;
          const int64_t n = nbase + c4 * 4;
          buf_store16f(ro, row_off(m, M, NR, n, 4), v);
        }
        wave_sync();
      });
      return;
    }
    constexpr int LD = WN + 8;           // bf16 staging [32][WN], padded rows
    constexpr int CPR = WN / 8;          // 16-byte chunks per row
    constexpr int RPP = 64 / CPR;        // rows per pass
    uint16_t* stg = reinterpret_cast<uint16_t*>(wstage);
    const int64_t ldo = args.reg[reg].ldo;
    const brsrc ro = make_rsrc(args.reg[reg].out, M * ldo * 2);
    if (!cols_ok) return;
    for4([&](auto jc) {
      constexpr int j = decltype(jc)::value;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const f32x4 a = quad(acc, q, j);
        u32x2 v;
        v[0] = pack_bf2(a[0], a[1]);
        v[1] = pack_bf2(a[2], a[3]);
        *reinterpret_cast<u32x2*>(stg + qrow(acc, q, lane) * LD + qcol(acc, q, lane)) = v;
      }
      wave_sync();
#pragma unroll
      for (int it = 0; it < 32 / RPP; ++it) {
        const int row = it * RPP + lane / CPR, c8 = lane % CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * LD + c8 * 8);
        const int64_t m = mw + j * 32 + row;
        const int64_t n = nbase + c8 * 8;
        buf_store16(ro, row_off(m, M, ldo, n, 2), v);
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
    const int64_t ld = args.ld_act;
    const brsrc eo = make_rsrc(args.e_out, M * ld * 2);
    const brsrc go = make_rsrc(args.g_out, M * ld * 2);
    const brsrc ho = make_rsrc(args.h_out, M * ld * 2);
    // with u_part: U_d = h Ad over this wavefront's 32 h columns (FusedU)
    const bool fuse_u = args.u_part != nullptr;
    FusedU<W2> fu;
    if (fuse_u) fu.init(args, nbase, NR, lane);
    if (cols_ok) {
      for4([&](auto jc) {
        constexpr int j = decltype(jc)::value;
#pragma unroll
        for (int q = 0; q < NQ / 2; ++q) {
          const f32x4 a = quad(acc, q, j), b = quad(acc, q + NQ / 2, j);  // gate, up
          u32x2 ev, gv, hv;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            ev[h] = pack_bf2(a[2 * h], a[2 * h + 1]);
            gv[h] = pack_bf2(b[2 * h], b[2 * h + 1]);
            float p0, p1;
            act_fwd<false>(ACT, lo_bf(ev[h]), p0);
            act_fwd<false>(ACT, hi_bf(ev[h]), p1);
            hv[h] = pack_bf2(p0 * lo_bf(gv[h]), p1 * hi_bf(gv[h]));
          }
          const int o = qrow(acc, q, lane) * LD + qcol(acc, q, lane);
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
          const int o = row * LD + c8 * 8;
          const uint32_t off = row_off(m, M, ld, n, 2);
          buf_store16(eo, off, *reinterpret_cast<const u32x4*>(stg + o));
          buf_store16(go, off, *reinterpret_cast<const u32x4*>(stg + ARR + o));
          buf_store16(ho, off, *reinterpret_cast<const u32x4*>(stg + 2 * ARR + o));
        }
        if (fuse_u) fu.template pass<j, LD>(stg + 2 * ARR, lane);
        wave_sync();
      });
    }
    // this tile's n index: 128 output columns per gate/up tile (a wavefront
    // past NR contributes zero sums: its h columns meet zero Ad^T rows)
    if (fuse_u) fu.template finish<epi_stage_bytes<WN, EPI>()>(args, wstage, mw, (nbase - 32 * wn) / 128, M, wn, lane);
  } else if constexpr (EPI == EPI_ACT1_FWD) {
    constexpr int LD = WN + 8;           // bf16 staging [2][32][WN]: u, h
    constexpr int ARR = 32 * LD;
    constexpr int CPR = WN / 8;
    constexpr int RPP = 64 / CPR;
    uint16_t* stg = reinterpret_cast<uint16_t*>(wstage);
    const int64_t ld = args.ld_act;
    const brsrc uo = make_rsrc(args.e_out, M * ld * 2);
    const brsrc ho = make_rsrc(args.h_out, M * ld * 2);
    // with u_part: U_d = h Ad over this wavefront's WN h columns (FusedU)
    const bool fuse_u = args.u_part != nullptr;
    FusedU<WN> fu;
    if (fuse_u) fu.init(args, nbase, NR, lane);
    if (cols_ok) {
      for4([&](auto jc) {
        constexpr int j = decltype(jc)::value;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const f32x4 a = quad(acc, q, j);
          u32x2 uv, hv;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uv[h] = pack_bf2(a[2 * h], a[2 * h + 1]);
            hv[h] = pack_bf2(relu2(lo_bf(uv[h])), relu2(hi_bf(uv[h])));
          }
          const int o = qrow(acc, q, lane) * LD + qcol(acc, q, lane);
          *reinterpret_cast<u32x2*>(stg + o) = uv;
          *reinterpret_cast<u32x2*>(stg + ARR + o) = hv;
        }
        wave_sync();
#pragma unroll
        for (int it = 0; it < 32 / RPP; ++it) {
          const int row = it * RPP + lane / CPR, c8 = lane % CPR;
          const int64_t m = mw + j * 32 + row;
          const int64_t n = nbase + c8 * 8;
          const int o = row * LD + c8 * 8;
          const uint32_t off = row_off(m, M, ld, n, 2);
          buf_store16(uo, off, *reinterpret_cast<const u32x4*>(stg + o));
          buf_store16(ho, off, *reinterpret_cast<const u32x4*>(stg + ARR + o));
        }
        if (fuse_u) fu.template pass<j, LD>(stg + ARR, lane);
        wave_sync();
      });
    }
    // this tile's n index: 256 output columns per tile
    if (fuse_u) fu.template finish<epi_stage_bytes<WN, EPI>()>(args, wstage, mw, (nbase - (int64_t)WN * wn) / 256, M, wn, lane);
  } else {
    // EPI_ACT_BWD (gated) or EPI_ACT1_BWD (ungated ReLU^2: du = dh phi'(u) into dg_out)
    //
    // With dA_part (fused adapter gradient of the next projection): h is
    // staged in LDS instead of stored, and h^T Pd over this wavefront's rows
    // is accumulated with 16x16x32 MFMAs (M = 16 columns of h, N = the 16
    // columns of Pd, K = 32 rows per pass), both operands read with the
    // transposing LDS read from row-major staging.  The two row groups of the
    // block are added in LDS and written as the block's m-tile slice.
    //
    // With rc_part (the rank-r products of the gradients written here): each
    // pass also stages its bf16 gradient rows dZ_p and, with 16x16x32 MFMAs,
    //  - adds U_p^T dZ_p over its rows the same way as h^T Pd (M = 16
    //    columns of dZ_p, N = the 16 columns of U_p, K = 32 rows);
    //  - forms dZ_p B_p^T over the wavefront's columns (M = 16 rows, N = the
    //    16 rows of B_p, K = 32 columns, dZ_p read K-contiguous), which the
    //    four wavefronts of the row group add in LDS in a fixed order (two
    //    block barriers per pass) and write as the tile's n-slice.
    constexpr bool GATED = EPI == EPI_ACT_BWD;
    constexpr int NP = GATED ? 2 : 1;    // gradients with fused rank-r products
    constexpr int LD = WN + 4;           // fp32 staging [32][WN]
    constexpr int CPR = WN / 8;          // 8-float groups per row
    constexpr int RPP = 64 / CPR;
    constexpr int PASSES = 32 / RPP;
    constexpr int HLD = WN + 8;          // bf16 row staging [32][WN] (h, dZ_p)
    constexpr int NCB = WN / 16;         // 16-column blocks of the fused products
    constexpr int EB = epi_stage_bytes<WN, EPI>();
    constexpr int R0 = bwd_region0<WN, EPI>();
    static_assert(WN == 64 || WN == 32, "row products take 32-column K blocks");
    float* stg = reinterpret_cast<float*>(wstage);
    uint16_t* zs = reinterpret_cast<uint16_t*>(wstage);  // dZ_p rows, once stg is read
    uint16_t* hs = reinterpret_cast<uint16_t*>(wstage + R0);
    uint16_t* pds = hs + 32 * HLD;       // Pd rows of the pass [32][16]
    uint16_t* us = pds + 32 * 16;        // U_p rows of the pass [NP][32][16]
    const lds_char* const hs_l = (const lds_char*)hs;
    const lds_char* const pds_l = (const lds_char*)pds;
    const lds_char* const zs_l = (const lds_char*)zs;
    const lds_char* const us_l = (const lds_char*)us;
    const bool fuse = args.dA_part != nullptr;
    const bool frc = args.rc_part[0] != nullptr;  // uniform over the block
    f32x4 dacc[NCB];
    f32x4 dbacc[NP][NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      dacc[cb] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < NP; ++p) dbacc[p][cb] = f32x4{0, 0, 0, 0};
    }
    const int64_t ld = args.ld_act;
    const brsrc ei = make_rsrc(args.e_in, M * ld * 2);
    const brsrc gi = make_rsrc(args.g_in, M * ld * 2);
    const brsrc dgo = make_rsrc(args.dg_out, M * ld * 2);
    const brsrc deo = make_rsrc(args.de_out, M * ld * 2);
    const brsrc ho = make_rsrc(args.h_out, M * ld * 2);
    const brsrc pdr = make_rsrc(args.pd, M * args.ldpd * 2);
    const brsrc ur = make_rsrc(args.rc_u, M * args.rc_ldu * 2);
    // B_p fragments of the wavefront's columns: lane l holds B_p[l % 16][n .. n + 7],
    // n = nbase + 32 kb + 8 (l / 16) (rows past the rank read zero)
    bf16x8 bfr[NP][WN / 32];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int kb = 0; kb < WN / 32; ++kb) {
        u32x4 v = u32x4{0, 0, 0, 0};
        if (frc && cols_ok) {
          const brsrc br = make_rsrc(args.rc_b[p], (int64_t)args.rc_R * args.rc_ldb * 2);
          v = buf_load16(br, (uint32_t)(((lane & 15) * args.rc_ldb + nbase + 32 * kb + 8 * (lane >> 4)) * 2));
        }
        bfr[p][kb] = __builtin_bit_cast(bf16x8, v);
      }
    // e, g of 32-row pass j (rows past M read zero, so h is zero there); the
    // loads of pass j + 1 are issued before pass j is computed, so each pass
    // waits for memory only as long as the previous pass's work does not cover
    u32x4 evn[PASSES], gvn[PASSES];
    auto load_eg = [&](int j) {
#pragma unroll
      for (int it = 0; it < PASSES; ++it) {
        const int row = it * RPP + lane / CPR, c8 = lane % CPR;
        const int64_t m = mw + j * 32 + row;
        const int64_t n = nbase + c8 * 8;
        const uint32_t off = row_off(m, M, ld, n, 2);
        evn[it] = buf_load16(ei, off);
        if constexpr (GATED) gvn[it] = buf_load16(gi, off);
      }
    };
    // a wavefront past NR leaves dacc and dbacc zero (those rows are not
    // written) and, with rc_part, takes part in every pass's barriers with
    // zero row products
    if (cols_ok || frc) {
      if (cols_ok) load_eg(0);
      for4([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        f32x4 pacc[NP][2];
#pragma unroll
        for (int p = 0; p < NP; ++p) pacc[p][0] = pacc[p][1] = f32x4{0, 0, 0, 0};
        if (cols_ok) {
#pragma unroll
          for (int q = 0; q < NQ; ++q)
            *reinterpret_cast<f32x4*>(stg + qrow(acc, q, lane) * LD + qcol(acc, q, lane)) = quad(acc, q, j);
          // Pd and U_p rows of this pass: lane l loads half l & 1 of row l / 2 (rows past M read zero)
          const int64_t mh = mw + j * 32 + (lane >> 1);
          u32x4 pv = u32x4{0, 0, 0, 0};
          if (fuse) pv = buf_load16(pdr, row_off(mh, M, args.ldpd, 8 * (lane & 1), 2));
          u32x4 uv[NP];
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            uv[p] = u32x4{0, 0, 0, 0};
            if (frc) uv[p] = buf_load16(ur, row_off(mh, M, args.rc_ldu, args.rc_uoff[p] + 8 * (lane & 1), 2));
          }
          u32x4 ev[PASSES], gv[PASSES];
#pragma unroll
          for (int it = 0; it < PASSES; ++it) {
            ev[it] = evn[it];
            if constexpr (GATED) gv[it] = gvn[it];
          }
          if constexpr (j < 3) load_eg(j + 1);
          wave_sync();
          f32x4 d0[PASSES], d1[PASSES];
#pragma unroll
          for (int it = 0; it < PASSES; ++it) {
            const int row = it * RPP + lane / CPR, c8 = lane % CPR;
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
              if constexpr (GATED) {
                const float g0 = lo_bf(gv[it][q]), g1 = hi_bf(gv[it][q]);
                float p0, s0, p1, s1;
                act_fwd_bwd<false>(ACT, e0, p0, s0);
                act_fwd_bwd<false>(ACT, e1, p1, s1);
                hv[q] = pack_bf2(p0 * g0, p1 * g1);
                dgv[q] = pack_bf2(dha * p0, dhb * p1);
                dev[q] = pack_bf2(dha * g0 * s0, dhb * g1 * s1);
              } else {
                hv[q] = pack_bf2(relu2(e0), relu2(e1));
                dgv[q] = pack_bf2(dha * relu2_grad(e0), dhb * relu2_grad(e1));
              }
            }
            const uint32_t off = row_off(m, M, ld, n, 2);
            buf_store16(dgo, off, dgv);
            if constexpr (GATED) buf_store16(deo, off, dev);
            if (!fuse) buf_store16(ho, off, hv);
            else *reinterpret_cast<u32x4*>(hs + row * HLD + c8 * 8) = hv;
            // every read of stg above precedes these writes in this wavefront's LDS order
            if (frc) {
              *reinterpret_cast<u32x4*>(zs + row * HLD + c8 * 8) = dgv;
              if constexpr (GATED) *reinterpret_cast<u32x4*>(zs + 32 * HLD + row * HLD + c8 * 8) = dev;
            }
          }
          if (fuse || frc) {
            if (fuse) *reinterpret_cast<u32x4*>(pds + (lane >> 1) * 16 + 8 * (lane & 1)) = pv;
            if (frc) {
#pragma unroll
              for (int p = 0; p < NP; ++p)
                *reinterpret_cast<u32x4*>(us + p * 512 + (lane >> 1) * 16 + 8 * (lane & 1)) = uv[p];
            }
            wave_sync();
            // lanes 16 g + 4 jj + q point at row 8 g + jj (+ 4), columns 4 q .. 4 q + 3 of a
            // 16-column block: lane 16 g + i receives column i of rows 8 g .. 8 g + 7
            const int g = lane >> 4, jj = (lane & 15) >> 2, q = lane & 3;
            if (fuse) {
              const bf16x8 pb = lds_read_tr8(pds_l + ((8 * g + jj) * 16 + 4 * q) * 2, 4 * 16 * 2);
#pragma unroll
              for (int cb = 0; cb < NCB; ++cb) {
                const bf16x8 ha = lds_read_tr8(hs_l + ((8 * g + jj) * HLD + 16 * cb + 4 * q) * 2, 4 * HLD * 2);
                dacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha, pb, dacc[cb], 0, 0, 0);
              }
            }
            if (frc) {
#pragma unroll
              for (int p = 0; p < NP; ++p) {
                const lds_char* const zp = zs_l + p * 32 * HLD * 2;
                const bf16x8 ub = lds_read_tr8(us_l + (p * 512 + (8 * g + jj) * 16 + 4 * q) * 2, 4 * 16 * 2);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                  const bf16x8 za = lds_read_tr8(zp + ((8 * g + jj) * HLD + 16 * cb + 4 * q) * 2, 4 * HLD * 2);
                  dbacc[p][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(za, ub, dbacc[p][cb], 0, 0, 0);
                }
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                  for (int kb = 0; kb < WN / 32; ++kb) {
                    const bf16x8 zr = __builtin_bit_cast(
                        bf16x8, lds_read16(zp + ((16 * rb + (lane & 15)) * HLD + 32 * kb + 8 * (lane >> 4)) * 2));
                    pacc[p][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zr, bfr[p][kb], pacc[p][rb], 0, 0, 0);
                  }
              }
            }
          }
        }
        if (frc) {
          // pacc[p][rb][v] = row 16 rb + 4 (lane / 16) + v, rank column lane % 16, over this
          // wavefront's columns; staged [p][32][16] fp32 in its h region (read above)
          float* const xs = reinterpret_cast<float*>(hs);
#pragma unroll
          for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
              for (int v = 0; v < 4; ++v) xs[p * 512 + (16 * rb + 4 * (lane >> 4) + v) * 16 + (lane & 15)] = pacc[p][rb][v];
          __syncthreads();
          // wavefront wn adds the row group's four wavefronts (ascending) for gradient wn / 2,
          // rows 16 (wn & 1) .. + 15 (gated), or rows 8 wn .. 8 wn + 7 (ungated, lanes < 32)
          const int p = GATED ? (wn >> 1) : 0;
          const int row = GATED ? 16 * (wn & 1) + (lane >> 2) : 8 * wn + ((lane >> 2) & 7);
          const int j4 = 4 * (lane & 3);
          const char* const g0 = wstage - wn * EB + R0;
          f32x4 s = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) s += *reinterpret_cast<const f32x4*>(g0 + w2 * EB + (p * 512 + row * 16 + j4) * 4);
          const int64_t m = mw + j * 32 + row;
          const int64_t tn = (nbase - (int64_t)WN * wn) / 256;
          if (m < M && (GATED || lane < 32)) *reinterpret_cast<f32x4*>(args.rc_rpart[p] + (tn * M + m) * 16 + j4) = s;
          __syncthreads();  // the h regions are rewritten by the next pass
        }
        wave_sync();
      });
    }
    if (fuse || frc) {
      // dacc[cb][v] = sum over this wavefront's 128 rows of h[., c] Pd[., lane % 16] (dbacc:
      // dZ_p[., c] U_p[., lane % 16]), c = 16 cb + 4 (lane / 16) + v.  Group 1 hands its
      // sums to group 0 through LDS.
      f32x4* red = reinterpret_cast<f32x4*>(wstage);
      if (wm == 1) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          red[cb * 64 + lane] = dacc[cb];
#pragma unroll
          for (int p = 0; p < NP; ++p) red[((1 + p) * NCB + cb) * 64 + lane] = dbacc[p][cb];
        }
      }
      __syncthreads();
      if (wm == 0 && cols_ok) {
        // the block's sums, staged [WN columns][16] (row pitch 20 floats) per product in this
        // wavefront's region 0 (its hand-off area is unused), then stored as 1 KB runs: the
        // wavefront's WN columns of a [., N, 16] slice are contiguous
        const f32x4* other = reinterpret_cast<const f32x4*>(wstage + 4 * EB);
        float* const tb = reinterpret_cast<float*>(wstage);
        constexpr int TP = 20, TB = WN * TP;
        static_assert((1 + NP) * TB * 4 <= EB, "sum staging exceeds the wavefront's region");
        const int64_t tm = mw / 256;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int o = (16 * cb + 4 * (lane >> 4) + v) * TP + (lane & 15);
            tb[o] = dacc[cb][v] + other[cb * 64 + lane][v];
#pragma unroll
            for (int p = 0; p < NP; ++p) tb[(1 + p) * TB + o] = dbacc[p][cb][v] + other[((1 + p) * NCB + cb) * 64 + lane][v];
          }
        wave_sync();
#pragma unroll
        for (int i = 0; i < WN / 16; ++i) {
          const int col = 16 * i + (lane >> 2), j4 = 4 * (lane & 3);
          const int64_t off = (tm * NR + nbase + col) * 16 + j4;
          if (fuse) *reinterpret_cast<f32x4*>(args.dA_part + off) = *reinterpret_cast<const f32x4*>(tb + col * TP + j4);
          if (frc) {
#pragma unroll
            for (int p = 0; p < NP; ++p)
              *reinterpret_cast<f32x4*>(args.rc_part[p] + off) =
                  *reinterpret_cast<const f32x4*>(tb + (1 + p) * TB + col * TP + j4);
          }
        }
      }
    }
  }
}

// NF4 level table of one block: the 16 products fl32(level_c * absmax)
// rounded to bf16, kept as two byte planes of four dwords (entry c is byte
// c % 4 of dword c / 4 of each plane).
struct Nf4Planes {
  uint32_t lo[4], hi[4];
};
__device__ __forceinline__ Nf4Planes nf4_planes(float absmax) {
  const float lv[16] = LORA_NF4_LEVELS_INIT;
  Nf4Planes p;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = pack_bf2(__fmul_rn(lv[4 * q], absmax), __fmul_rn(lv[4 * q + 1], absmax));
    const uint32_t b = pack_bf2(__fmul_rn(lv[4 * q + 2], absmax), __fmul_rn(lv[4 * q + 3], absmax));
    p.lo[q] = __builtin_amdgcn_perm(b, a, 0x06040200u);
    p.hi[q] = __builtin_amdgcn_perm(b, a, 0x07050301u);
  }
  return p;
}
// Byte k of the result is plane entry (code k): sel holds the codes' low 3
// bits, fsel = k + 4 * (bit 3 of code k) picks entries 0-7 or 8-15.
__device__ __forceinline__ uint32_t nf4_lookup(const uint32_t (&pl)[4], uint32_t sel, uint32_t fsel) {
  const uint32_t a = __builtin_amdgcn_perm(pl[1], pl[0], sel);
  const uint32_t b = __builtin_amdgcn_perm(pl[3], pl[2], sel);
  return __builtin_amdgcn_perm(b, a, fsel);
}
// 8 codes of one dword (element 2j in the high nibble of byte j, element
// 2j + 1 in its low nibble) -> 8 bf16, in element order (NAT) or in the order
// 0, 2, 4, 6, 1, 3, 5, 7, which saves the four final interleaving permutes.
template <bool NAT>
__device__ __forceinline__ u32x4 nf4_decode8(uint32_t w, const Nf4Planes& p) {
  const uint32_t se = (w >> 4) & 0x07070707u, fe = ((w >> 5) & 0x04040404u) | 0x03020100u;
  const uint32_t so = w & 0x07070707u, fo = ((w >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t le = nf4_lookup(p.lo, se, fe), he = nf4_lookup(p.hi, se, fe);
  const uint32_t lo = nf4_lookup(p.lo, so, fo), ho = nf4_lookup(p.hi, so, fo);
  const uint32_t e01 = __builtin_amdgcn_perm(he, le, 0x05010400u), e23 = __builtin_amdgcn_perm(he, le, 0x07030602u);
  const uint32_t o01 = __builtin_amdgcn_perm(ho, lo, 0x05010400u), o23 = __builtin_amdgcn_perm(ho, lo, 0x07030602u);
  u32x4 r;
  if constexpr (NAT) {
    r[0] = __builtin_amdgcn_perm(o01, e01, 0x05040100u);
    r[1] = __builtin_amdgcn_perm(o01, e01, 0x07060302u);
    r[2] = __builtin_amdgcn_perm(o23, e23, 0x05040100u);
    r[3] = __builtin_amdgcn_perm(o23, e23, 0x07060302u);
  } else {
    r[0] = e01;
    r[1] = e23;
    r[2] = o01;
    r[3] = o23;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Dense weights.  8 wavefronts in two groups of 4, one wavefront of each
// group on every SIMD, working in alternating phases separated by barriers:
// while group 0 runs a cluster of MFMAs (one K step: 64 of 16x16x32, or 32
// of 32x32x16 in the NF4 kernels) on fragments already in its registers,
// group 1 reads the fragments of its next cluster from LDS, and then the
// roles swap -- the SIMD's matrix unit always has one wavefront feeding it and
// LDS latency never sits between two MFMAs.  Each wavefront owns a 128x64
// sub-tile (32 accumulators of 16x16, or 8 of 32x32); group g covers tile
// rows 128 g .. 128 g + 127.
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
//
// NF4 weights.  The weight group loads, per K step, the packed codes (8 KB)
// and for each of the tile's 256 blocks the dword holding its int8 scale code
// and its fp32 second-level scale (1 KB each) into a 3-slot code ring, three
// steps ahead.  Both groups unpack, during their MFMA clusters, half of every
// block each into a 2-slot bf16 weight ring with the dense layout: group 1
// the upper 32 elements of step t+2 in Y(t), group 0 the lower 32 elements of
// step t+1 in X(t).  A weight slot is rewritten only after both groups have
// read it, so two slots suffice, and 30 KB of code ring fit beside them.  The
// adapter K tile is dense and is loaded like a dense weight tile.
// ---------------------------------------------------------------------------
constexpr int NTH8 = 512;
constexpr int SLOT_BYTES = 32768;
constexpr int A_SLOTS = 2;
constexpr int W_RING = A_SLOTS * SLOT_BYTES;  // weight ring after the activation ring
constexpr int LDS_BYTES = 5 * SLOT_BYTES;     // dense: 3 weight slots; NF4: 2 + code ring
constexpr int HALF_BYTES = 16384;
constexpr int CODE_RING = W_RING + 2 * SLOT_BYTES;
constexpr int CODE_SLOT = 10240;  // codes 8 KB | scale-code dwords 1 KB | fp32 scales 1 KB
constexpr int SPARE = CODE_RING + 3 * CODE_SLOT;  // target of the stores of an idle unpack
constexpr int SPARE_BYTES = 2048;
static_assert(SPARE + SPARE_BYTES <= LDS_BYTES, "NF4 code ring exceeds LDS");

template <int BKIND, bool DUAL, int EPI, bool NF4, int ACT>
__global__ __launch_bounds__(NTH8, 1) void gemm_kernel(const GemmArgs args) {
  static_assert(!(DUAL && BKIND == B_NT && NF4), "NF4 gate/up tiles read forward (NN) weights");
  __shared__ __attribute__((aligned(1024))) char smem_raw[LDS_BYTES];
  lds_char* const lds = (lds_char*)smem_raw;
  // timing build only: real-time stamps (entry, K loop start, K loop end) and
  // the shader clock at entry
  unsigned long long tstamp[3] = {0, 0, 0}, tclock0 = 0;
  if constexpr (kBlockTiming) {
    tstamp[0] = __builtin_amdgcn_s_memrealtime();
    tclock0 = __builtin_amdgcn_s_memtime();
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lane_id = lane;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int wm = wave >> 2, wn = wave & 3;                    // wm: the group

  int tm, tn;
  // split-K: blocks below ksplit_t0 compute tiles 0 .. t0-1 whole; block
  // t0 + u computes K part u / ns of tile t0 + u % ns (ns = ntiles - t0), so
  // only the tiles past the last full round of the grid are split
  const int ntiles = (int)(args.ntile_m * args.ntile_n);
  int tile = (int)blockIdx.x, kp = -1;
  if (!NF4 && args.ksplit > 1 && tile >= args.ksplit_t0) {
    const int u = tile - args.ksplit_t0, ns = ntiles - args.ksplit_t0;
    kp = u / ns;
    tile = args.ksplit_t0 + (u - kp * ns);
  }
  tile_coords(tile, ntiles, (int)args.ntile_m, (int)args.ntile_n, args.group, tm, tn);
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

  int KT = 0, KN = 0;  // all K steps; NF4 steps (the NF4 segments come first)
  int nseg_nf4 = 0;
  for (int s = 0; s < args.nseg; ++s) {
    const int k = (int)(args.seg[s].K / BK);
    KT += k;
    if (NF4 && args.seg[s].b[reg][0].codes != nullptr) {
      KN += k;
      ++nseg_nf4;
    }
  }
  // this block's K steps [k_begin, k_begin + KT) (dense split-K only)
  int k_begin = 0;
  if (!NF4 && kp >= 0) {
    const int kall = KT;
    k_begin = (int)((int64_t)kp * kall / args.ksplit);
    KT = (int)((int64_t)(kp + 1) * kall / args.ksplit) - k_begin;
  }

  // ---- loads: 8 blocks of 1 KB per wavefront and step ----
  // K-contiguous block q = 8 wn + i holds rows 8 q + lane / 8; its row r has
  // swz(r) = (lane / 8) ^ kc_i(i), kc_i(i) = 0 (dense) or i (NF4), so lane
  // takes logical chunk (lane % 8) ^ (lane / 8) ^ kc_i(i).
  // NN block q' = 8 (wn & 1) + i of half wn >> 1 holds K rows 4 q' + lane / 16,
  // lane takes logical chunk (lane % 16) ^ 4 (lane / 16) (dense) or the NF4
  // swizzle of its row (the adapter tile of an NF4 GEMM).
  constexpr bool M16 = !NF4;  // 16x16x32 MFMA blocks (fragment reads below)
  const auto kc_i = [](int i) { return M16 ? 0 : i; };
  const int kc_row = wn * 64 + (lane >> 3);
  const int kc_x = (lane & 7) ^ (lane >> 3);
  const int nn_row = (wn & 1) * 32 + (lane >> 4);
  const int nn_chunk = (lane & 15) ^ (4 * ((lane >> 4) & 3));
  // Each group walks the K steps with a load cursor of its own (group 0: the
  // activation tiles; group 1: the weight tiles, or an NF4 segment's codes and
  // scales).  The current segment's window is kept in scalar registers and
  // advanced by one K step per load; the segment table in the kernel
  // arguments is read only when a segment starts, not at the head of every
  // read phase.
  int lseg = 0, lsteps = 0, lk0 = 0;
  const char* lp = nullptr;  // dense operand at the next K step
  int64_t ln = 0;            // bytes from lp to the end of its window
  uint32_t lld2 = 0;         // row pitch in bytes
  int64_t lstep = 0;         // bytes lp advances per K step
  const uint8_t* lcodes = nullptr;  // NF4 segment
  const int8_t* lq8 = nullptr;
  const float* ls2 = nullptr;
  int64_t lnumel = 0;
  int lwcols = 0;
  // every field is assigned on every call (selects, no early exits), so the
  // cursor stays in scalar registers
  // Dense kernels: the per-lane source offset of this wavefront's 8 loads is
  // the same for all of them (the swizzle r & 7 of a K-contiguous block
  // depends only on lane / 8, and a dense NN block needs none per load), so it
  // is formed once per segment and held in a register; the loads differ only
  // in their scalar offset.  Forming it per load pair took a v_mul_lo_u32 and
  // three more vector instructions from every read phase (measured: config 2
  // -1.3%).
  uint32_t dma_base = 0;
  auto cur_begin = [&]() {
    const GemmSeg& S = args.seg[lseg];
    const BSrc& B = S.b[reg][DUAL ? (wn >> 1) : 0];
    lsteps = (int)(S.K / BK);
    lk0 = 0;
    const char* pw;
    int64_t nw, sw;
    if constexpr (BKIND == B_NT) {
      // gate/up tiles: rows 0..127 of the tile are 128 gate columns, rows
      // 128..255 the same up columns (column group wn / 2 of the loader)
      const int64_t row0 = DUAL ? tnl * 128 : tnl * 256;
      pw = static_cast<const char*>(B.p) + row0 * B.ld * 2;
      nw = (NR - row0) * B.ld * 2;
      sw = BK * 2;
    } else {
      const int64_t ncol0 = DUAL ? tnl * 128 : tnl * 256 + (wn >> 1) * 128;
      pw = static_cast<const char*>(B.p) + ncol0 * 2;
      nw = ((S.K - 1) * B.ld + NR - ncol0) * 2;
      sw = (int64_t)BK * B.ld * 2;
    }
    const bool act = wm == 0;
    lp = act ? static_cast<const char*>(S.A) + m0 * S.lda * 2 : pw;
    ln = act ? (M - m0) * S.lda * 2 : nw;
    lld2 = (uint32_t)((act ? S.lda : B.ld) * 2);
    lstep = act ? (int64_t)BK * 2 : sw;
    if constexpr (M16) {
      // the loaders' row and chunk (kc_row / kc_x, nn_row / nn_chunk), formed
      // from the thread index here so that none of them stays live in the loop
      const int l = (int)threadIdx.x & 63;
      const int kr = (BKIND == B_NT && DUAL && !act ? (wn & 1) * 64 : wn * 64) + (l >> 3);
      const int r = (act || BKIND == B_NT) ? kr : (wn & 1) * 32 + (l >> 4);
      const int c = (act || BKIND == B_NT) ? ((l & 7) ^ (l >> 3)) : ((l & 15) ^ (4 * ((l >> 4) & 3)));
      dma_base = (uint32_t)r * lld2 + (uint32_t)(c << 4);
    }
    if constexpr (NF4) {  // NF4 segment (group 1): codes and scales
      lcodes = B.codes;
      lq8 = B.q8;
      ls2 = B.s2;
      lwcols = (int)B.wcols;
      lnumel = (BKIND == B_NN ? S.K : NR) * B.wcols;
    }
  };
  cur_begin();
  // skip to this block's first K step (split-K)
  for (int sk = k_begin; sk > 0;) {
    const int n = sk < lsteps ? sk : lsteps;
    lp += n * lstep;
    ln -= n * lstep;
    lk0 += n * BK;
    lsteps -= n;
    sk -= n;
    if (lsteps == 0 && lseg + 1 < args.nseg) {
      ++lseg;
      cur_begin();
    }
  }
  auto advance = [&]() {
    lp += lstep;
    ln -= lstep;
    lk0 += BK;
    if (--lsteps == 0 && lseg + 1 < args.nseg) {
      ++lseg;
      cur_begin();
    }
  };
  // The tile of one K step is 8 loads of 1 KB per wavefront; issue_a and
  // issue_w issue loads i0 .. i1 - 1 of them (constants once the callers'
  // loops are unrolled), and the caller advances the cursor once all 8 are
  // out.  In the K loop the read phase issues them two at a time after each
  // K slice's fragment reads (read's `between`), which keeps the LDS read
  // and the vector-memory queues busy together; at the Llama-3-8B MLP shape
  // this measured 1.2% less step time than all 8 after the reads.
  auto issue_a = [&](int slot, int i0, int i1) {  // group 0: activation tile of the next step
    const uint32_t dst = lds_addr(lds) + slot * SLOT_BYTES + wn * 8 * 1024;
    if constexpr (M16) {
      const i32x4 ra = rsrc_words(lp, ln);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i >= i0 && i < i1) dma16(ra, dma_base, dst + i * 1024, (uint32_t)(8 * i) * lld2);
      return;
    }
    // NF4 kernels (per-load swizzle terms): opaque copies keep the per-lane
    // terms from being expanded per load and hoisted out of the K loop (8 live
    // offsets would not fit)
    int x = kc_x, r = kc_row;
    asm volatile("" : "+v"(x), "+v"(r));
    const i32x4 ra = rsrc_words(lp, ln);
    const uint32_t base = (uint32_t)r * lld2;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i >= i0 && i < i1) dma16(ra, base + (uint32_t)((x ^ kc_i(i)) << 4), dst + i * 1024, (uint32_t)(8 * i) * lld2);
  };
  auto issue_w = [&](int slot, int i0, int i1) {  // group 1: (dense) weight tile of the next step
    const uint32_t wslot = lds_addr(lds) + W_RING + slot * SLOT_BYTES;
    const i32x4 rb = rsrc_words(lp, ln);
    if constexpr (M16) {
      const uint32_t dst = BKIND == B_NT ? wslot + wn * 8 * 1024 : wslot + (wn >> 1) * HALF_BYTES + (wn & 1) * 8 * 1024;
      const uint32_t step = BKIND == B_NT ? 8 : 4;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i >= i0 && i < i1) dma16(rb, dma_base, dst + i * 1024, (uint32_t)(step * i) * lld2);
    } else if constexpr (BKIND == B_NT) {
      // source row in the loader's column group (gate/up tiles: wn & 1 picks
      // the 64-row half); the LDS row and its swizzle are those of the tile
      int x = kc_x, r = DUAL ? (wn & 1) * 64 + (lane >> 3) : kc_row;
      asm volatile("" : "+v"(x), "+v"(r));
      const uint32_t base = (uint32_t)r * lld2;
      const uint32_t dst = wslot + wn * 8 * 1024;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i >= i0 && i < i1) dma16(rb, base + (uint32_t)((x ^ kc_i(i)) << 4), dst + i * 1024, (uint32_t)(8 * i) * lld2);
    } else if constexpr (!NF4) {
      int nr = nn_row, nc = nn_chunk;
      asm volatile("" : "+v"(nr), "+v"(nc));
      const uint32_t base = (uint32_t)nr * lld2 + (uint32_t)(nc << 4);
      const uint32_t dst = wslot + (wn >> 1) * HALF_BYTES + (wn & 1) * 8 * 1024;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i >= i0 && i < i1) dma16(rb, base, dst + i * 1024, (uint32_t)(4 * i) * lld2);
    } else {
      // the dense adapter tile of an NF4 GEMM, in the NF4 swizzle: load i
      // covers rows nn_row + 4 i, whose swizzle alternates with i & 1
      int nr = nn_row, nc = lane & 15;
      asm volatile("" : "+v"(nr), "+v"(nc));
      const uint32_t b0 = (uint32_t)nr * lld2 + (uint32_t)((nc ^ nn_swz<true>(nr)) << 4);
      const uint32_t b1 = (uint32_t)nr * lld2 + (uint32_t)((nc ^ nn_swz<true>(nr + 4)) << 4);
      const uint32_t dst = wslot + (wn >> 1) * HALF_BYTES + (wn & 1) * 8 * 1024;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i >= i0 && i < i1) dma16(rb, (i & 1) ? b1 : b0, dst + i * 1024, (uint32_t)(4 * i) * lld2);
    }
  };
  // a whole tile, then the cursor
  auto load_a = [&](int slot) {
    issue_a(slot, 0, 8);
    advance();
  };
  auto load_w = [&](int slot) {
    issue_w(slot, 0, 8);
    advance();
  };

  // ---- NF4: code staging and unpacking ----
  // Block j (0..63) of wavefront column wn; its first element sits at
  //   NN: weight row k0 + 32 (wn & 1) + j / 2, column c0 + 64 (j & 1)
  //       (c0: first column of the tile's half wn / 2),
  //   NT: weight row (= output column) 256 tnl + 64 wn + j, column k0.
  // Returns its flat element index, or a value past every NF4 array for
  // columns (NN) or rows (NT) outside the region, so its loads read zero.
  auto nf4_flat = [&](int wcols, int k0, int j) -> uint32_t {
    if constexpr (BKIND == B_NN) {
      const int col = (DUAL ? (int)tnl * 128 : (int)tnl * 256 + 128 * (wn >> 1)) + 64 * (j & 1);
      const int row = k0 + 32 * (wn & 1) + (j >> 1);
      return col < (int)NR ? (uint32_t)row * (uint32_t)wcols + (uint32_t)col : 0xffffff80u;
    } else {
      const int row = (int)tnl * 256 + 64 * wn + j;
      return row < (int)NR ? (uint32_t)row * (uint32_t)wcols + (uint32_t)k0 : 0xffffff80u;
    }
  };
  auto nf4_src = [&](const GemmSeg& S) -> const BSrc& { return S.b[reg][DUAL ? (wn >> 1) : 0]; };
  // group 1: codes and scales of the next NF4 step into code slot `slot`
  auto issue_codes = [&](int slot) {
    const i32x4 rc = rsrc_words(lcodes, lnumel / 2);
    const i32x4 rq = rsrc_words(lq8, lnumel / 64);
    const i32x4 rs = rsrc_words(ls2, lnumel / NF4_GROUP * 4);
    const uint32_t cs = lds_addr(lds) + CODE_RING + slot * CODE_SLOT;
    int l = lane;
    asm volatile("" : "+v"(l));
    // codes of block b at cs + 32 b: lane l of load j takes half l & 1 of block 64 wn + 32 j + l / 2
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t f = nf4_flat(lwcols, lk0, 32 * j + (l >> 1));
      dma16(rc, (f >> 1) + 16 * (l & 1), cs + 2048 * wn + 1024 * j);
    }
    // lane l: block 64 wn + l; the aligned dword holding its scale code, and its fp32 scale
    const uint32_t f = nf4_flat(lwcols, lk0, l);
    dma4(rq, (f >> 6) & ~3u, cs + 8192 + 256 * wn);
    dma4(rs, (f >> 14) << 2, cs + 9216 + 256 * wn);
    advance();
  };
  // each group walks the NF4 steps it unpacks with a cursor of its own
  int dseg = 0, dk0 = 0;
  // unpack half h (elements 32 h .. 32 h + 31) of block 64 wn + lane from code
  // slot cslot into weight slot wslot.  Without `live` (no step left to
  // unpack) the same work runs on stale codes and its stores go to 2 KB of
  // otherwise unused LDS, so the call has no branch and shares one
  // scheduling region with the MFMA cluster it is interleaved with.
  // The unpack is split in two.  unpack_fetch (in a read phase, where the
  // wavefront waits for LDS at the barrier anyway) reads the block's 32 codes
  // from the code ring and rebuilds its absmax from the scale code, the
  // second-level scale and the mean; unpack_store (interleaved with an MFMA
  // cluster) builds the level table, decodes and stores into the weight ring,
  // with no load, so no wait for LDS or scalar memory stalls the MFMAs.
  struct UnpackIn {
    u32x4 w;       // 32 codes
    float absmax;  // the block's reconstructed absmax
  };
  auto unpack_fetch = [&](int cslot, int h, bool live) -> UnpackIn {
    const GemmSeg& S = args.seg[dseg < nseg_nf4 ? dseg : nseg_nf4 - 1];
    const BSrc& B = nf4_src(S);
    // uniform: a scalar load (a vector load would make the compiler wait for
    // the global -> LDS loads in flight)
    const float mu = *(const __attribute__((address_space(4))) float*)(uintptr_t)B.mu;
    const lds_char* cs = lds + CODE_RING + cslot * CODE_SLOT;
    // opaque copy: keeps the per-lane terms below from being hoisted out of
    // the K loop, where they would stay live through the read phases
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int b = 64 * wn + lane;
    UnpackIn in;
    in.w = lds_read16(cs + 32 * b + 16 * h);
    const uint32_t q8w = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(cs + 8192 + 4 * b);
    const float s2 = *reinterpret_cast<const __attribute__((address_space(3))) float*>(cs + 9216 + 4 * b);
    // byte of the scale code inside its aligned dword: block index mod 4
    // (block index = (row wcols + col) / 64 with col a multiple of 64)
    uint32_t qb;
    if constexpr (BKIND == B_NN) {
      const uint32_t row = (uint32_t)(dk0 + 32 * (wn & 1)) + (uint32_t)(lane >> 1);
      qb = row * (uint32_t)(B.wcols >> 6) + (uint32_t)(lane & 1) +
           (uint32_t)(DUAL ? tnl * 2 : tnl * 4 + 2 * (wn >> 1));
    } else {
      qb = (uint32_t)((int)tnl * 256 + 64 * wn + lane) * (uint32_t)(B.wcols >> 6) + (uint32_t)(dk0 >> 6);
    }
    const int8_t q8 = (int8_t)(q8w >> (8 * (qb & 3)));
    in.absmax = nf4_absmax(q8, s2, mu);
    const int nk0 = dk0 + BK;
    const bool wrap = nk0 >= (int)S.K;
    dseg = live && wrap ? dseg + 1 : dseg;
    dk0 = live ? (wrap ? 0 : nk0) : dk0;
    return in;
  };
  // Without `live` (no step left to unpack) the same work runs on stale codes
  // and its stores go to 2 KB of otherwise unused LDS, so the call has no
  // branch and shares one scheduling region with the MFMA cluster.
  auto unpack_store = [&](const UnpackIn& in, int wslot, int h, bool live) {
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int b = 64 * wn + lane;
    const Nf4Planes pl = nf4_planes(in.absmax);
    lds_char* const wt = lds + (live ? W_RING + wslot * SLOT_BYTES : SPARE);
    const int omask = live ? 0x7fffffff : SPARE_BYTES - 1;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // NN tiles: the 8 columns of each chunk in the order 0, 2, 4, 6, 1, 3, 5, 7
      // (restored in the accumulators by restore_cols); NT tiles: K order
      const u32x4 v = nf4_decode8<BKIND != B_NN>(in.w[d], pl);
      int off;
      if constexpr (BKIND == B_NN) {
        const int k = 32 * (wn & 1) + (lane >> 1);
        const int c = 8 * (lane & 1) + 4 * h + d;
        off = (wn >> 1) * HALF_BYTES + k * 256 + ((c ^ nn_swz<true>(k)) << 4);
      } else {
        const int c = 4 * h + d;
        off = b * 128 + ((c ^ swz<false>(b)) << 4);
      }
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(wt + (off & omask)) = v;
    }
  };

  // ---- fragment reads ----
  // Dense kernels run 16x16x32 MFMA blocks, NF4 kernels 32x32x16 (file
  // header).  fa holds the weight (A) fragments of one K step and fb the
  // activation (B) fragments: fa[4 ks + i], fb[8 ks + j] over two K slices ks
  // of 32 (16x16x32), fa[2 ks + i], fb[4 ks + j] over four K slices of 16
  // (32x32x16).
  // NN weights, 32x32x16: lane s of read h (0, 1) of K slice ks points at K row
  //   16 ks + 8 (g >> 1) + 4 h + (s & 15) / 4 and columns nb + 16 (g & 1) + 4 (s & 3), g = s / 16
  // (rows 4 h apart; in the NF4 swizzle the two reads' chunk positions differ).
  // NN weights, 16x16x32: lane s of read h of K slice ks points at K row
  //   32 ks + 8 (s / 16) + 4 h + (s & 15) / 4 and columns nb + 4 (s & 3) of its 16-column
  // fragment.  Fragment i = 2 p + e starts at column nb_p + 16 e, whose chunk index is that
  // of nb_p plus 2 e; bit 1 of the chunk index is clear in nb_p's and in the dense swizzle,
  // so e adds 32 bytes to fa_nn[p].
  int fa_nn[2], fa_nn4[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int half = DUAL ? i : (wn >> 1);
    if constexpr (M16) {
      const int nb = DUAL ? wn * 32 : (wn & 1) * 64 + 32 * i;
      const int n = nb + 4 * (lane & 3);
      const int k0 = 8 * (lane >> 4) + ((lane & 15) >> 2);  // K row of read h = 0 in slice 0
      fa_nn[i] = half * HALF_BYTES + k0 * 256 + (((n >> 3) ^ nn_swz<false>(k0)) * 16) + (lane & 1) * 8;
      fa_nn4[i] = 0;
    } else {
      const int nb = DUAL ? wn * 32 : (wn & 1) * 64 + 32 * i;
      const int g = lane >> 4;
      const int n = nb + 16 * (g & 1) + 4 * (lane & 3);
      const int k0 = 8 * (g >> 1) + ((lane & 15) >> 2);  // K row of read h = 0 in slice 0
      fa_nn[i] = half * HALF_BYTES + k0 * 256 + (((n >> 3) ^ nn_swz<NF4>(k0)) * 16) + (lane & 1) * 8;
      fa_nn4[i] = half * HALF_BYTES + (k0 + 4) * 256 + (((n >> 3) ^ nn_swz<NF4>(k0 + 4)) * 16) + (lane & 1) * 8;
    }
  }
  // K-contiguous tiles, 32x32x16: row r0 + 32 j (r0 = first row of the sub-tile + lane % 32)
  // has swz = swz(r0) ^ 4 (j & 1), so chunk 2 ks + lane / 32 sits at
  // (2 ks ^ 4 (j & 1)) ^ x with x = (lane / 32) ^ swz(r0): four per-lane offsets
  // cover every (ks, j); the row term is an immediate.
  auto kc_offsets = [&](int r0, int (&o)[4]) {
    const int x = (lane >> 5) ^ swz<false>(r0);
#pragma unroll
    for (int y = 0; y < 4; ++y) o[y] = r0 * 128 + (((2 * y) ^ x) * 16);
  };
  // K-contiguous tiles, 16x16x32: lane l reads row r0 + 16 b + l % 16 (r0 a multiple of 16),
  // chunk 4 ks + l / 16, stored at that chunk ^ (l % 16 & 7) (the dense swizzle depends on
  // the row's low 3 bits only): one per-lane offset per K slice, o[ks]; the row term 16 b
  // is an immediate.
  auto kc16_offsets = [&](int r0, int (&o)[4]) {
    const int l16 = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) o[ks] = (r0 + l16) * 128 + ((((4 * ks) | (lane >> 4)) ^ swz<true>(l16)) * 16);
    o[2] = o[3] = 0;
  };
  const auto kc16_at = [](int ks, int) { return ks; };
  int ao[4];
  if constexpr (M16) kc16_offsets(wm * 128, ao);
  else kc_offsets(wm * 128 + (lane & 31), ao);
  // NT weights: the wavefront's 64 tile rows from wn * 64; in gate/up tiles the
  // 32 gate rows from wn * 32 and the up rows 128 below them, whose swizzle is
  // the same
  int bo[4];
  if constexpr (BKIND == B_NT) {
    if constexpr (M16) kc16_offsets(DUAL ? wn * 32 : wn * 64, bo);
    else kc_offsets(DUAL ? wn * 32 + (lane & 31) : wn * 64 + (lane & 31), bo);
  }

  bf16x8 fa[8], fb[16];
  // between(c) runs after each quarter c (0..3) of the step's fragment reads
  auto read = [&](int aslot, int wslot, auto&& between) {
    const lds_char* const at = lds + aslot * SLOT_BYTES;
    const lds_char* const wt = lds + W_RING + wslot * SLOT_BYTES;
    if constexpr (M16) {
      // quarter 2 ks + h: weight fragments 2 h, 2 h + 1 and activation
      // fragments 4 h .. 4 h + 3 of K slice ks
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int i = 2 * h + e;
            if constexpr (BKIND == B_NN)
              fa[4 * ks + i] = lds_read_tr8(wt + fa_nn[h] + 32 * e + (32 * ks) * 256, 4 * 256);
            else if constexpr (DUAL)
              fa[4 * ks + i] =
                  __builtin_bit_cast(bf16x8, lds_read16(wt + bo[kc16_at(ks, e)] + 2048 * e + 16384 * h));
            else
              fa[4 * ks + i] = __builtin_bit_cast(bf16x8, lds_read16(wt + bo[kc16_at(ks, i)] + 2048 * i));
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int j = 4 * h + jj;
            fb[8 * ks + j] = __builtin_bit_cast(bf16x8, lds_read16(at + ao[kc16_at(ks, j)] + 2048 * j));
          }
          between(2 * ks + h);
        }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if constexpr (BKIND == B_NN) {
            if constexpr (NF4)
              fa[2 * ks + i] = lds_read_tr8(wt + fa_nn[i] + (16 * ks) * 256, wt + fa_nn4[i] + (16 * ks) * 256);
            else
              fa[2 * ks + i] = lds_read_tr8(wt + fa_nn[i] + (16 * ks) * 256, 4 * 256);
          } else {
            const int y = DUAL ? ks : ((2 * ks) ^ (4 * (i & 1))) >> 1;
            fa[2 * ks + i] = __builtin_bit_cast(bf16x8, lds_read16(wt + bo[y] + i * (DUAL ? 128 : 32) * 128));
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int y = ((2 * ks) ^ (4 * (j & 1))) >> 1;
          fb[4 * ks + j] = __builtin_bit_cast(bf16x8, lds_read16(at + ao[y] + j * 32 * 128));
        }
        between(ks);
      }
    }
  };
  const auto nothing = [](int) {};

  std::conditional_t<M16, f32x4[4][8], f32x16[2][4]> acc;
  if constexpr (M16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  }
  // the MFMA phase runs at raised wavefront priority, so the SIMD's other
  // wavefront (in its read phase) cannot delay the MFMA issue
  auto mma_body = [&]() {
    if constexpr (M16) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[4 * ks + i], fb[8 * ks + j], acc[i][j], 0, 0, 0);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[2 * ks + i], fb[4 * ks + j], acc[i][j], 0, 0, 0);
    }
  };
  auto mma = [&]() {
    __builtin_amdgcn_s_setprio(1);
    mma_body();
    __builtin_amdgcn_s_setprio(0);
  };
  // NF4 NN tiles store each 8-column group of the weight tile in the order
  // 0, 2, 4, 6, 1, 3, 5, 7, so accumulator registers 4k .. 4k + 3 hold, in lanes
  // 0-31, columns 8k + 0, 2, 4, 6 and in lanes 32-63 columns 8k + 1, 3, 5, 7
  // (natural: 8k + 0..3 and 8k + 4..7).  Exchanging the upper lane half of
  // registers 4k, 4k + 1 with the lower lane half of registers 4k + 2, 4k + 3
  // (v_permlane32_swap) and renaming restores the natural order.  It runs once,
  // after the K loop: the dense adapter tile of these GEMMs comes packed in the
  // same column order (the pack job's perm8).
  auto restore_cols = [&]() {
    if constexpr (!M16) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            float n0, n1, n2, n3;
            swap_lane_halves(acc[i][j][4 * k], acc[i][j][4 * k + 2], n0, n1);
            swap_lane_halves(acc[i][j][4 * k + 1], acc[i][j][4 * k + 3], n2, n3);
            acc[i][j][4 * k] = n0;
            acc[i][j][4 * k + 1] = n1;
            acc[i][j][4 * k + 2] = n2;
            acc[i][j][4 * k + 3] = n3;
          }
    }
  };
  // MFMA cluster with the store half of an unpack interleaved: about five of
  // its vector instructions after each MFMA (its inputs are in registers).
  // Unlike the dense clusters it runs at normal priority and the NF4 read
  // phases run raised: the unpack's vector instructions would otherwise hold
  // back the address arithmetic and loads of the SIMD's other wavefront,
  // whose read phase then ends later (measured: config-4 step -3%).
  auto mma_unpack = [&](const UnpackIn& in, int wslot, int h, bool live) {
    mma_body();
    unpack_store(in, wslot, h, live);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
  };

  // ---- phases.  Every wavefront passes 2 + 2 KT barriers. ----
  //   prologue  g0 loads A 0, 1   g1 loads W 0, 1; each waits for step 0 | barrier
  //             g0 reads step 0                                         | barrier
  //   step t    X: g0 MFMA t, waits for A t+1
  //                g1 reads step t, loads W t+2, waits for W t+1        | barrier
  //             Y: g0 reads step t+1, loads A t+2
  //                g1 MFMA t                                            | barrier
  // A t+2 goes to activation slot t & 1 after its last read (g1, X(t));
  // W t+2 goes to weight slot (t+2) % 3, last read in X(t-1).
  auto phase_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  // phase-timing build only: stamp k of K step t (see phase_times)
#ifdef LORA_PHASE_TIMING
  unsigned long long pst[5] = {0, 0, 0, 0, 0}, pnext = 0;
#endif
  auto pstamp = [&](int t, auto kc) {
#ifdef LORA_PHASE_TIMING
    constexpr int k = decltype(kc)::value;
    __builtin_amdgcn_sched_barrier(0);
    const unsigned long long x = __builtin_amdgcn_s_memtime();
    if (t == kPhaseStep) pst[k] = x;
    if (k == 0 && t == kPhaseStep + 1) pnext = x;
    __builtin_amdgcn_sched_barrier(0);
#else
    (void)t;
    (void)kc;
#endif
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  using P4 = std::integral_constant<int, 4>;
  if constexpr (!NF4) {
    if (wm == 0) {
      load_a(0);
      if (KT > 1) {
        load_a(1);
        __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): A 0 is in
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      phase_end();
      read(0, 0, nothing);
      phase_end();
      if constexpr (kBlockTiming) tstamp[1] = __builtin_amdgcn_s_memrealtime();
      for (int t = 0; t < KT; ++t) {
        pstamp(t, P0{});
        mma();
        pstamp(t, P1{});
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): A t+1 is in
        pstamp(t, P2{});
        phase_end();
        pstamp(t, P3{});
        // fragment reads lead: they are the phase's critical path
        if (t + 2 < KT) {
          read((t + 1) & 1, (t + 1) % 3, [&](int ks) { issue_a(t & 1, 2 * ks, 2 * ks + 2); });
          advance();
        } else if (t + 1 < KT) {
          read((t + 1) & 1, (t + 1) % 3, nothing);
        }
        pstamp(t, P4{});
        phase_end();
      }
      if constexpr (kBlockTiming) tstamp[2] = __builtin_amdgcn_s_memrealtime();
    } else {
      load_w(0);
      if (KT > 1) {
        load_w(1);
        __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): W 0 is in
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      phase_end();
      phase_end();
      int ws = 0;  // weight slot of step t
      for (int t = 0; t < KT; ++t) {
        const int ws2 = ws == 0 ? 2 : ws - 1;  // (t + 2) % 3
        pstamp(t, P0{});
        if (t + 2 < KT) {
          read(t & 1, ws, [&](int ks) { issue_w(ws2, 2 * ks, 2 * ks + 2); });
          advance();
          __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): W t+1 is in (W t+2 may still fly)
        } else {
          read(t & 1, ws, nothing);
          __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        pstamp(t, P1{});
        phase_end();
        pstamp(t, P2{});
        mma();
        pstamp(t, P3{});
        phase_end();
        ws = ws == 2 ? 0 : ws + 1;
      }
    }
  } else {
    // ---- NF4 phases (steps t < KN unpacked, the adapter step t = KN loaded) ----
    //   P1  g0 loads A 0, 1             g1 loads codes 0, 1, 2, waits for codes 0   | barrier
    //   P2  g0 unpacks W 0 (lower half)  g1 unpacks W 0 (upper), waits for codes 1
    //       g0 waits for A 0                                                         | barrier
    //   P3  g0 reads step 0, fetches W 1 (lower)
    //       g1 unpacks W 1 (upper) or loads the adapter W 1                          | barrier
    //   X(t)  g0 MFMA t, stores W t+1 (lower), waits for A t+1
    //         g1 reads step t, loads codes t+3, waits for codes t+2 (and adapter W),
    //         fetches W t+2 (upper)                                                  | barrier
    //   Y(t)  g0 reads step t+1, loads A t+2, fetches W t+2 (lower)
    //         g1 MFMA t, stores W t+2 (upper) or loads the adapter W t+2            | barrier
    // Weight slot of step t: t & 1; code slot: t % 3.  A fetch reads codes that
    // its own wavefront waited for (g1) or that a barrier has published (g0).
    const bool lora_step = KT > KN;  // the last step is the dense adapter tile
    if (wm == 0) {
      load_a(0);
      if (KT > 1) load_a(1);
      phase_end();
      {
        const UnpackIn u = unpack_fetch(0, 0, true);
        unpack_store(u, 0, 0, true);
      }
      if (KT > 1) wait_vmcnt<8>();
      else wait_vmcnt<0>();
      phase_end();
      read(0, 0, nothing);
      UnpackIn nx = unpack_fetch(1, 0, 1 < KN);  // W 1 (lower): code slot 1
      phase_end();
      if constexpr (kBlockTiming) tstamp[1] = __builtin_amdgcn_s_memrealtime();
      int cs2 = 2;  // code slot of step t + 2
      for (int t = 0; t < KT; ++t) {
        pstamp(t, P0{});
        mma_unpack(nx, (t + 1) & 1, 0, t + 1 < KN);
        pstamp(t, P1{});
        wait_vmcnt<0>();  // A t+1 is in
        pstamp(t, P2{});
        phase_end();
        pstamp(t, P3{});
        __builtin_amdgcn_s_setprio(1);
        if (t + 1 < KT) read((t + 1) & 1, (t + 1) & 1, nothing);
        if (t + 2 < KT) load_a(t & 1);
        nx = unpack_fetch(cs2, 0, t + 2 < KN);
        __builtin_amdgcn_s_setprio(0);
        pstamp(t, P4{});
        phase_end();
        cs2 = cs2 == 2 ? 0 : cs2 + 1;
      }
      if constexpr (kBlockTiming) tstamp[2] = __builtin_amdgcn_s_memrealtime();
      if constexpr (BKIND == B_NN) restore_cols();
    } else {
      issue_codes(0);
      if (KN > 1) issue_codes(1);
      if (KN > 2) {
        issue_codes(2);
        wait_vmcnt<8>();
      } else if (KN > 1) {
        wait_vmcnt<4>();
      } else {
        wait_vmcnt<0>();
      }
      phase_end();
      {
        const UnpackIn u = unpack_fetch(0, 1, true);
        unpack_store(u, 0, 1, true);
      }
      if (KN > 2) wait_vmcnt<4>();
      else wait_vmcnt<0>();
      phase_end();
      if (KN > 1) {
        const UnpackIn u = unpack_fetch(1, 1, true);
        unpack_store(u, 1, 1, true);
      } else if (lora_step) {
        load_w(1);
      }
      phase_end();
      int cs0 = 0;  // code slot of step t (= that of step t + 3)
      for (int t = 0; t < KT; ++t) {
        const int cs2 = cs0 == 0 ? 2 : cs0 - 1;  // (t + 2) % 3
        pstamp(t, P0{});
        __builtin_amdgcn_s_setprio(1);
        if (t + 3 < KN) {
          read(t & 1, t & 1, nothing);
          issue_codes(cs0);
          wait_vmcnt<4>();  // codes t+2 are in (codes t+3 may still fly)
        } else {
          read(t & 1, t & 1, nothing);
          wait_vmcnt<0>();
        }
        const UnpackIn nx = unpack_fetch(cs2, 1, t + 2 < KN);
        __builtin_amdgcn_s_setprio(0);
        pstamp(t, P1{});
        phase_end();
        pstamp(t, P2{});
        mma_unpack(nx, t & 1, 1, t + 2 < KN);
        if (lora_step && t + 2 == KN) load_w(t & 1);
        pstamp(t, P3{});
        phase_end();
        cs0 = cs0 == 2 ? 0 : cs0 + 1;
      }
      if constexpr (BKIND == B_NN) restore_cols();
    }
  }

#ifdef LORA_PHASE_TIMING
  if ((wave == 0 || wave == 4) && lane == 0 && blockIdx.x < 64u) {
    constexpr int fam = (NF4 ? 4 : 0) + ((EPI == EPI_ACT_FWD || EPI == EPI_ACT1_FWD) ? 0
                                         : (EPI == EPI_ACT_BWD || EPI == EPI_ACT1_BWD) ? 1
                                         : BKIND == B_NT ? 2 : 3);
    unsigned long long* d = phase_times[fam][blockIdx.x][wave >> 2];
    d[0] = pst[0];
    d[1] = pst[1];
    d[2] = pst[2];
    d[3] = pst[3];
    d[4] = pst[4];
    d[5] = pnext;
    d[6] = (unsigned long long)(unsigned)KT;
    d[7] = (unsigned long long)gridDim.x;
  }
#endif
  // epilogue staging: a private region per wavefront (operand slots are no longer read)
  constexpr int EB = epi_stage_bytes<64, EPI>();
  static_assert(8 * EB <= LDS_BYTES, "epilogue staging exceeds LDS");
  char* const wstage = smem_raw + wave * EB;
  const int64_t mw = m0 + wm * 128;
  const int64_t nbase = DUAL ? tnl * 128 + wn * 32 : tnl * 256 + wn * 64;
  run_epilogue_w<64, DUAL, EPI, ACT>(acc, wstage, args, reg, mw, nbase, NR, M, lane, wm, wn, kp);
#ifdef LORA_BLOCK_TIMING
  {
    const unsigned long long t3 = __builtin_amdgcn_s_memrealtime(), c3 = __builtin_amdgcn_s_memtime();
    unsigned int hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    constexpr int fam = (NF4 ? 4 : 0) + ((EPI == EPI_ACT_FWD || EPI == EPI_ACT1_FWD) ? 0
                                         : (EPI == EPI_ACT_BWD || EPI == EPI_ACT1_BWD) ? 1
                                         : BKIND == B_NT ? 2 : 3);
    if (wave == 0 && lane == 0 && blockIdx.x < (unsigned)kTimedBlocks) {
      unsigned long long* d = block_times[fam][blockIdx.x];
      d[0] = tstamp[0];
      d[1] = tstamp[1];
      d[2] = tstamp[2];
      d[3] = t3;
      d[4] = tclock0;
      d[5] = c3;
      d[6] = (unsigned long long)hw | ((unsigned long long)xcc << 32);
      d[7] = (unsigned long long)gridDim.x | ((unsigned long long)(unsigned)KT << 32);
    }
  }
#endif
}

// Sum of the K parts of the split tiles t0 .. ntiles-1 (tile order as in the
// GEMM): 32 blocks per tile, each 8 rows of 256 columns, 8 columns per thread.
__global__ void ksplit_reduce_kernel(const float* part, int ks, int64_t M, int64_t N, uint16_t* out, int64_t ldo,
                                     int t0, int ntm, int ntn, int G) {
  const int tile = t0 + (int)(blockIdx.x >> 5);
  int tm, tn;
  tile_coords(tile, ntm * ntn, ntm, ntn, G, tm, tn);
  const int64_t m = (int64_t)tm * 256 + (blockIdx.x & 31) * 8 + (threadIdx.x >> 5);
  const int64_t n = (int64_t)tn * 256 + (threadIdx.x & 31) * 8;
  if (m >= M || n >= N) return;  // N is a multiple of 8
  const int64_t e = m * N + n;
  f32x4 a = *reinterpret_cast<const f32x4*>(part + e), b = *reinterpret_cast<const f32x4*>(part + e + 4);
  for (int k = 1; k < ks; ++k) {
    a += *reinterpret_cast<const f32x4*>(part + (int64_t)k * M * N + e);
    b += *reinterpret_cast<const f32x4*>(part + (int64_t)k * M * N + e + 4);
  }
  const u32x4 v = {pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3])};
  *reinterpret_cast<u32x4*>(out + m * ldo + n) = v;
}

template <int BKIND, bool DUAL, int EPI, bool NF4, int ACT = 0>
hipError_t launch(const GemmArgs& a, hipStream_t st) {
  const int64_t nt = a.ntile_m * a.ntile_n;
  const int64_t nb = a.ksplit > 1 && !NF4 ? a.ksplit_t0 + (nt - a.ksplit_t0) * a.ksplit : nt;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<BKIND, DUAL, EPI, NF4, ACT>), dim3((unsigned)nb), dim3(NTH8), 0, st, a);
  return hipGetLastError();
}

template <bool NF4>
hipError_t launch_family(const GemmArgs& a, hipStream_t st) {
  if (a.bkind == B_NN) {
    if (a.epi == EPI_ACT_FWD)
      return a.act == LORA_ACT_SWIGLU ? launch<B_NN, true, EPI_ACT_FWD, NF4, LORA_ACT_SWIGLU>(a, st)
                                      : launch<B_NN, true, EPI_ACT_FWD, NF4, LORA_ACT_GEGLU_TANH>(a, st);
    if (a.epi == EPI_ACT1_FWD) return launch<B_NN, false, EPI_ACT1_FWD, NF4>(a, st);
    return launch<B_NN, false, EPI_STORE, NF4>(a, st);
  }
  if constexpr (!NF4) {  // forward GEMMs over K-contiguous weights (dense only)
    if (a.epi == EPI_ACT_FWD)
      return a.act == LORA_ACT_SWIGLU ? launch<B_NT, true, EPI_ACT_FWD, false, LORA_ACT_SWIGLU>(a, st)
                                      : launch<B_NT, true, EPI_ACT_FWD, false, LORA_ACT_GEGLU_TANH>(a, st);
    if (a.epi == EPI_ACT1_FWD) return launch<B_NT, false, EPI_ACT1_FWD, false>(a, st);
  } else {
    if (a.epi == EPI_ACT_FWD || a.epi == EPI_ACT1_FWD) return hipErrorInvalidValue;
  }
  if (a.epi == EPI_ACT_BWD)
    return a.act == LORA_ACT_SWIGLU ? launch<B_NT, false, EPI_ACT_BWD, NF4, LORA_ACT_SWIGLU>(a, st)
                                    : launch<B_NT, false, EPI_ACT_BWD, NF4, LORA_ACT_GEGLU_TANH>(a, st);
  if (a.epi == EPI_ACT1_BWD) return launch<B_NT, false, EPI_ACT1_BWD, NF4>(a, st);
  return launch<B_NT, false, EPI_STORE, NF4>(a, st);
}

}  // namespace

int64_t gemm_tile_cols(bool bf16, bool dual) {
  if (bf16) return dual ? 128 : 256;
  return dual ? 32 : 64;
}
int64_t gemm_tile_rows(bool bf16) { return bf16 ? 256 : 64; }

hipError_t launch_ksplit_reduce(const GemmArgs& a, hipStream_t st) {
  const int64_t nsplit = a.ntile_m * a.ntile_n - a.ksplit_t0;
  if (a.ksplit <= 1 || nsplit <= 0) return hipSuccess;
  hipLaunchKernelGGL(ksplit_reduce_kernel, dim3((unsigned)(nsplit * 32)), dim3(256), 0, st, a.kpart, a.ksplit, a.M,
                     a.reg[0].N, static_cast<uint16_t*>(a.reg[0].out), a.reg[0].ldo, a.ksplit_t0, (int)a.ntile_m,
                     (int)a.ntile_n, a.group);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t st) {
  return a.nf4 ? launch_family<true>(a, st) : launch_family<false>(a, st);
}

}  // namespace lora

#ifdef LORA_PHASE_TIMING
// Phase-timing build only: copies the phase records ([8 families][64 blocks]
// [2 groups][8] unsigned 64-bit words, see phase_times) to host memory `out`
// of `bytes` bytes (at least their size).  Synchronises the device first.
// Returns a HIP error code (0 on success).
extern "C" int lora_phase_times(void* out, size_t bytes) {
  if (out == nullptr || bytes < sizeof(lora::phase_times)) return (int)hipErrorInvalidValue;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return (int)e;
  return (int)hipMemcpyFromSymbol(out, HIP_SYMBOL(lora::phase_times), sizeof(lora::phase_times), 0,
                                  hipMemcpyDeviceToHost);
}
#endif

#ifdef LORA_BLOCK_TIMING
// Timing build only: copies the per-block records ([8 families][8192 blocks][8]
// unsigned 64-bit words, see block_times) to host memory `out` of `bytes`
// bytes (at least their size).  Synchronises the device first.  Returns a HIP
// error code (0 on success).
extern "C" int lora_block_times(void* out, size_t bytes) {
  if (out == nullptr || bytes < sizeof(lora::block_times)) return (int)hipErrorInvalidValue;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return (int)e;
  return (int)hipMemcpyFromSymbol(out, HIP_SYMBOL(lora::block_times), sizeof(lora::block_times), 0,
                                  hipMemcpyDeviceToHost);
}
#endif
