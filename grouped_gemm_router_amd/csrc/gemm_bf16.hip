// gemm_bf16.hip -- grouped GEMM on bf16 MFMA for gfx950, one launch over
// ragged groups.
//
// "DeepGEMM walkthrough" §4.2 (load tiles, multiply on the matrix cores,
// accumulate in registers, write back), §4.3 (many GEMMs of different M in
// one launch over an expert-contiguous layout), §5.2 (double buffering --
// here deeper LDS rings -- so loads overlap the multiplies), §5.3 (rows past a
// group's end are masked); "Dense GEMM to TP MoE" §2.1-2.3 (grouped, not
// batched: N and K shared, M_i ragged; expert sizes stay on the GPU).
//
// Design (CDNA4, 64-wide waves):
//   * output tile BM x 256 (BM = 256, or 128 / 64 for the last, partial
//     tile of a group), K step 32, 4 or 8 waves in a 2 x (NW/2) grid; each
//     wave owns BM/2 x (256/(NW/2)) = MI x NB blocks of
//     v_mfma_f32_32x32x16_bf16;
//   * operand tiles move HBM/L2 -> LDS with global_load_lds_dwordx4 (no
//     staging registers), each step waits only for its own data (vmcnt) and
//     meets the other waves at a plain s_barrier (no release fence, which
//     would drain every in-flight load);
//   * both operands move as whole 128-byte row pieces (two K steps): the
//     TCP sends one L2 request per line touched, and the request count is
//     what bounds this kernel.  A (activations) runs through a ring of two
//     such double stages (2 x 32 KB), each refilled (odd steps) as soon as
//     its second step has been read, so it lands two steps ahead of use; B
//     (weights) through three (3 x 32 KB), refilled on even steps, four to
//     five steps ahead.  Measured (gate/up / down): on the Mixtral shapes
//     all-64-byte rings 1.91 / 1.08 ms, 64-byte A with 128-byte B 1.75 /
//     0.96, then 128-byte A 1.67 / 0.91 (DeepSeek shapes 3.40 -> 3.20 /
//     2.00 -> 1.97); a 2-stage ring for both operands 2.25 / 1.39 (too little
//     in flight), and 64-deep steps with one barrier each were slower on the
//     Mixtral shapes.  The two rings fill the 160 KB of LDS;
//   * a row is 8 pieces of 16 bytes, piece p of row r at slot p ^ ((r >> 1)
//     & 7): the DMA writes whole rows and the MFMA fragment reads (16 rows x
//     one piece per phase) hit distinct banks;
//   * fragments are double buffered in registers and the stage barrier sits
//     in the middle of a stage, so the next stage's first fragments are read
//     while this stage's second half of MFMAs runs; the LDS reads are
//     scheduled two per MFMA at the start of each 16-deep step;
//   * SwiGLU: the B tile holds 128 gate rows then the 128 matching up rows;
//     each wave's columns cover matching gate and up rows, so the epilogue
//     pairs silu(gate) * up in registers;
//   * the tile scheduler reads the device offsets array (no host round trip
//     of expert sizes); tiles are taken in an order that keeps all XCDs on
//     one expert at a time (the tile order in moe_internal.h), except that
//     SwiGLU launches over fine-grained experts deal each expert's column
//     tiles to one XCD;
//   * ragged tails: A rows past the group end are loaded (clamped to the
//     tile's last row) and multiplied but never stored;
//   * weight rows sit ldb >= K elements apart (B[g][n][k] at (g N + n) ldb
//     + k): a power-of-two row pitch puts the 128-byte pieces that a tile
//     reads at one K offset on few HBM channels, so callers streaming such
//     weights from HBM pad them (measured alone: decode-size gate/up, 8 KB
//     rows, 403 -> 321 us with 256 bytes of padding; DeepSeek-shape down,
//     4 KB rows, 1852 -> 1709 us; the Mixtral-shape GEMMs, fed from L2 and
//     the MALL, unchanged);
//   * the last, partial round of tiles (fewer tiles than half the CUs) is
//     cut along K into S slices when a workspace is given: each slice writes
//     an fp32 partial tile to the workspace and a second small kernel adds the
//     S partials in slice order (deterministic) and applies the epilogue, so
//     the chip is not three-quarters idle for the last tile's duration.
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int BM_MAX = 256, BN = 256, BK = 32;
constexpr int PIECES = BK / 8;             // 16-byte pieces per operand row and stage
constexpr int PIECES_B = 2 * PIECES;       // 128-byte row pieces covering two stages
constexpr int SLOTS_A2MAX = BM_MAX * PIECES_B; // 16-byte slots per A double stage (32 KB)
constexpr int SLOTS_B2 = BN * PIECES_B;    // 16-byte slots per B double stage (32 KB)

__device__ __forceinline__ int swzb(int row, int p) { return p ^ ((row >> 1) & 7); }

constexpr long long kLastLevelCacheBytes = 256LL << 20;  // the MI355X MALL

// B-tile row of wave column wn (of NWN), 32-row block nb
template <bool SWIGLU, int NWN>
__device__ __forceinline__ int b_row(int wn, int nb) {
  if (SWIGLU) {
    constexpr int per = 128 / NWN;  // gate rows per wave column
    constexpr int half = per / 32;  // 32-row blocks in each half
    return ((nb >= half) ? 128 : 0) + wn * per + (nb % half) * 32;
  }
  return wn * (BN / NWN) + nb * 32;
}

// LDS-direct load: lane i's SZ bytes from g land at l + i * SZ
template <int SZ>
__device__ __forceinline__ void dma_to_lds(const uint16_t *g, u32x4 *l) {
  if constexpr (SZ == 16)
    __builtin_amdgcn_global_load_lds((const void *)g, (lds_void *)l, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds((const void *)g, (lds_void *)l, 4, 0, 0);
}

template <int MI, int NB>
struct Frag {
  bf16x8 a[MI];
  bf16x8 b[NB];
};

// live: the wave's 32-row blocks that hold rows of the group (wave-uniform;
// MI except in the short SwiGLU tiles that skip); blocks past the group end
// are neither read from LDS nor multiplied
template <bool SWIGLU, int MI, int NB, int NWN>
__device__ __forceinline__ void read_frag(Frag<MI, NB> &f, const u32x4 *tA, const u32x4 *tB,
                                          int ks, int par, int wm, int wn, int fr, int fh,
                                          int live) {
  const int pc = ks * 2 + fh;
  const int pb = par * PIECES + pc;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    if (mi >= live) break;
    const int r = wm * (MI * 32) + mi * 32 + fr;
    f.a[mi] = __builtin_bit_cast(bf16x8, tA[r * PIECES_B + swzb(r, pb)]);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = b_row<SWIGLU, NWN>(wn, nb) + fr;
    f.b[nb] = __builtin_bit_cast(bf16x8, tB[r * PIECES_B + swzb(r, pb)]);
  }
}

template <int MI, int NB>
__device__ __forceinline__ void mfma_frag(f32x16 (&acc)[MI][NB], const Frag<MI, NB> &f,
                                          int live) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
    if (mi < live)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mi][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[nb], acc[mi][nb], 0, 0, 0);
}

// scheduling hint: two LDS reads after each of the first MFMAs, so the
// next 16-deep step's fragments are requested early in this step's MFMAs
// (measured against one read per MFMA: Mixtral-shape down 0.90 -> 0.88 ms,
// gate/up unchanged; all reads first or three per MFMA were no better)
template <int NMFMA, int NREAD>
__device__ __forceinline__ void interleave_mfma_ds_read() {
#pragma unroll
  for (int i = 0; i < (NREAD + 1) / 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - (NREAD + 1) / 2, 0);
}

// Split of the tail: workspace layout and plan.  The workspace holds a
// header (n_split, S), the position of every split tile, then the fp32
// partial tiles [split tile][slice][BM_MAX][BN] (B-tile column order).
constexpr int kSplitMax = 8;         // slices per tile at most
constexpr int kSplitMinSteps = 32;   // K steps per slice at least (K/S >= 1024)
constexpr size_t kPartialFloats = (size_t)BM_MAX * BN;

__host__ __device__ inline size_t split_desc_offset() { return 64; }
__host__ __device__ inline size_t split_partial_offset(int cus) {
  return (split_desc_offset() + 16 * (size_t)cus + 255) / 256 * 256;
}

// Slices per tail tile: 1 (no split) unless the last round holds at most
// half as many tiles as there are CUs; then the largest S <= kSplitMax with
// S * rem <= cus, KT a multiple of 4 S (the rings advance 4 steps at a time)
// and at least kSplitMinSteps steps per slice.
__host__ __device__ inline int split_slices(int total, int cus, int KT) {
  const int rem = total % cus;
  if (rem == 0 || 2 * rem > cus) return 1;
  int S = kSplitMax;
  while (S > 1 && (S * rem > cus || KT % (4 * S) != 0 || KT / S < kSplitMinSteps)) S >>= 1;
  return S;
}

// One output tile of height BM (rows [tile.m0, tile.mend), at most BM of
// them) over K steps [kbeg/BK, kbeg/BK + KT), through the A and B LDS rings.
// part == nullptr: the epilogue writes C; otherwise the raw fp32 accumulator
// goes to part[(m - m0) * BN + B-tile row] (a K-slice of a split tile).
// SKIP: the tile may be shorter than BM; a wave's 32-row blocks wholly past
// the group end are not computed (their accumulators stay zero and their
// rows are never stored).
template <int BM, bool SWIGLU, bool OUT_F32, int NW, bool SKIP>
__device__ __forceinline__ void run_tile(const Tile &tile, const uint16_t *__restrict__ A,
                                         const uint16_t *__restrict__ B,
                                         const uint16_t *__restrict__ B2, void *__restrict__ C,
                                         int rows, int N, int K, int ldb, int kbeg, int KT,
                                         float *__restrict__ part, u32x4 *sA0, u32x4 *sA1,
                                         u32x4 *sB0, u32x4 *sB1, u32x4 *sB2, bool nt_store) {
  constexpr int NWN = NW / 2;                 // wave columns (2 wave rows)
  constexpr int MI = BM / 64;                 // 32-row blocks per wave
  constexpr int NB = (BN / NWN) / 32;         // 32-column blocks per wave
  constexpr int SLOTS_A2 = BM * PIECES_B;     // 16-byte slots per A double stage
  constexpr int IA = SLOTS_A2 / NW / 64;      // A DMA instructions per wave per double stage
  constexpr int IB = SLOTS_B2 / NW / 64;      // B DMA instructions per wave per double stage
  constexpr int NM = MI * NB;                 // MFMAs per 16-deep step
  constexpr int NR = MI + NB;                 // fragment reads per 16-deep step
  static_assert(IA >= 1 && IB >= 1, "tile too small for the wave count");

  // the wave index is uniform: scalar, so LDS destinations (M0) and block
  // bases need no per-use readfirstlane
  const int tid = threadIdx.x, lane = lane_id(),
            wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wv / NWN, wn = wv % NWN;
  int live = MI;
  if (SKIP) {
    const int hv = __builtin_amdgcn_readfirstlane(tile.mend - tile.m0 - wm * (MI * 32));
    live = hv <= 0 ? 0 : min(MI, (hv + 31) / 32);
  }

  // DMA sources: wave wv fills slots [wv*SLOTS/NW, +SLOTS/NW) of each
  // operand double stage, 64 slots per instruction; slot s holds piece
  // swzb(row, s % 8) of row s / 8.
  const uint16_t *gb[IB];
  const size_t goff = (size_t)tile.g * N * ldb + kbeg;
  const uint16_t *ga[IA];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int sl = wv * (SLOTS_A2 / NW) + i * 64 + lane;
    const int r = sl / PIECES_B;
    // rows past the tile's last row repeat that row (one address, so the
    // loads of a dead row block coalesce and hit the L1) and are never
    // stored; measured against clamping to the buffer's last row, which
    // loads the next group's rows (DeepSeek shapes, ~143 rows per 256-row
    // tile): gate/up 3059 -> 3002 us, down 1876 -> 1838 us; Mixtral down
    // 872 -> 861 us
    const int m = min(tile.m0 + r, tile.mend - 1);
    ga[i] = A + (size_t)m * K + kbeg + swzb(r, sl % PIECES_B) * 8;
  }
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    const int sl = wv * (SLOTS_B2 / NW) + i * 64 + lane;
    const int r = sl / PIECES_B;
    const int p = swzb(r, sl % PIECES_B);
    if (SWIGLU) {
      const int n = tile.nt * 128 + (r & 127);
      gb[i] = (r < 128 ? B : B2) + goff + (size_t)n * ldb + p * 8;
    } else {
      gb[i] = B + goff + (size_t)(tile.nt * 256 + r) * ldb + p * 8;
    }
  }
  // LDS destinations of lane 0, in 16-byte units
  const int dma_a = wv * (SLOTS_A2 / NW);
  const int dma_b = wv * (SLOTS_B2 / NW);
#define MOE_ISSUE_A(dA, k0)                                                                \
  _Pragma("unroll") for (int i = 0; i < IA; ++i)                                          \
    __builtin_amdgcn_global_load_lds((const void *)(ga[i] + (k0)),                        \
                                     (lds_void *)((dA) + dma_a + i * 64), 16, 0, 0);
#define MOE_ISSUE_B(dB, k0)                                                                \
  _Pragma("unroll") for (int i = 0; i < IB; ++i)                                          \
    __builtin_amdgcn_global_load_lds((const void *)(gb[i] + (k0)),                        \
                                     (lds_void *)((dB) + dma_b + i * 64), 16, 0, 0);

  f32x16 acc[MI][NB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};
  const int fr = lane & 31, fh = lane >> 5;

  const int KT2 = KT / 2;  // double stages
  MOE_ISSUE_B(sB0, 0);
  MOE_ISSUE_A(sA0, 0);
  MOE_ISSUE_B(sB1, 2 * BK);
  MOE_ISSUE_A(sA1, 2 * BK);
  wait_vmcnt<IA + IB>();  // A and B double stage 0 landed
  stage_barrier();
  Frag<MI, NB> f0, f1;
  read_frag<SWIGLU, MI, NB, NWN>(f0, sA0, sB0, 0, 0, wm, wn, fr, fh, live);

  // One stage s: A from double-stage slot (s / 2) % 2, B from slot (s / 2) %
  // 3, half s % 2.  The barrier in the middle makes stage s+1 visible.  An
  // odd s has just read the second half of its A slot: its wait also covers
  // this wave's LDS reads, and after the barrier the slot takes A double
  // stage (s + 3) / 2.  An even s frees B slot (s/2 + 2) % 3 (read last in
  // stage s-1) and refills it with double stage s/2 + 2.  Loads are issued
  // in the order A(d), B(d+1), A(d+1), B(d+2), ...: an odd s needs A and B
  // double stage (s+1)/2, after which only B((s+1)/2 + 1) was issued (IB
  // loads may stay in flight); an even s needs nothing new (IB + IA).  Past
  // the end the last double stage is re-loaded into slots nobody reads, so
  // the counts never change.
#define MOE_STAGE(tA, tB, tp, nA, nB, np, s, ODD, dA, dB)                                   \
  read_frag<SWIGLU, MI, NB, NWN>(f1, tA, tB, 1, tp, wm, wn, fr, fh, live);                   \
  mfma_frag<MI, NB>(acc, f0, live);                                                           \
  interleave_mfma_ds_read<NM, NR>();                                                          \
  if (ODD) { wait_vmcnt_lgkm0<IB>(); } else { wait_vmcnt<IB + IA>(); }                        \
  stage_barrier();                                                                            \
  if (ODD) { MOE_ISSUE_A(dA, min(((s) + 3) / 2, KT2 - 1) * 2 * BK); }                         \
  else { MOE_ISSUE_B(dB, min((s) / 2 + 2, KT2 - 1) * 2 * BK); }                               \
  read_frag<SWIGLU, MI, NB, NWN>(f0, nA, nB, 0, np, wm, wn, fr, fh, live);                   \
  mfma_frag<MI, NB>(acc, f1, live);                                                           \
  interleave_mfma_ds_read<NM, NR>();

// stage s: A slot (s/2)%2, B slot (s/2)%3, half s%2; odd s refills A slot
// ((s+3)/2)%2 (the one just read), even s refills B slot (s/2+2)%3
#define MOE_STAGES_0_3(kt)                                         \
  MOE_STAGE(sA0, sB0, 0, sA0, sB0, 1, (kt), 0, sA0, sB2)           \
  MOE_STAGE(sA0, sB0, 1, sA1, sB1, 0, (kt) + 1, 1, sA0, sB2)       \
  MOE_STAGE(sA1, sB1, 0, sA1, sB1, 1, (kt) + 2, 0, sA1, sB0)       \
  MOE_STAGE(sA1, sB1, 1, sA0, sB2, 0, (kt) + 3, 1, sA1, sB0)
#define MOE_STAGES_4_7(kt)                                         \
  MOE_STAGE(sA0, sB2, 0, sA0, sB2, 1, (kt) + 4, 0, sA0, sB1)       \
  MOE_STAGE(sA0, sB2, 1, sA1, sB0, 0, (kt) + 5, 1, sA0, sB1)       \
  MOE_STAGE(sA1, sB0, 0, sA1, sB0, 1, (kt) + 6, 0, sA1, sB2)       \
  MOE_STAGE(sA1, sB0, 1, sA0, sB1, 0, (kt) + 7, 1, sA1, sB2)
#define MOE_STAGES_8_11(kt)                                        \
  MOE_STAGE(sA0, sB1, 0, sA0, sB1, 1, (kt) + 8, 0, sA0, sB0)       \
  MOE_STAGE(sA0, sB1, 1, sA1, sB2, 0, (kt) + 9, 1, sA0, sB0)       \
  MOE_STAGE(sA1, sB2, 0, sA1, sB2, 1, (kt) + 10, 0, sA1, sB1)      \
  MOE_STAGE(sA1, sB2, 1, sA0, sB0, 0, (kt) + 11, 1, sA1, sB1)

  int kt = 0;
  for (; kt + 12 <= KT; kt += 12) {
    MOE_STAGES_0_3(kt)
    MOE_STAGES_4_7(kt)
    MOE_STAGES_8_11(kt)
  }
  if (kt + 4 <= KT) {  // KT % 12 is 0, 4 or 8
    MOE_STAGES_0_3(kt)
    if (kt + 8 <= KT) {
      MOE_STAGES_4_7(kt)
    }
  }
  wait_vmcnt<0>();  // no LDS-direct load may still be landing when the tile ends
#undef MOE_STAGES_0_3
#undef MOE_STAGES_4_7
#undef MOE_STAGES_8_11
#undef MOE_STAGE
#undef MOE_ISSUE_A
#undef MOE_ISSUE_B

  // epilogue.  32x32 accumulator layout: lane holds column lane%32, and
  // register r holds row 8*(r/4) + 4*(lane/32) + r%4.
  const int col = lane & 31, rbase = 4 * (lane >> 5);
  if (part != nullptr) {  // a K-slice of a split tile: raw fp32 partials
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mt = wm * (MI * 32) + mi * 32 + 8 * (r >> 2) + rbase + (r & 3);
          if (tile.m0 + mt < tile.mend)
            part[(size_t)mt * BN + b_row<SWIGLU, NWN>(wn, nb) + col] = acc[mi][nb][r];
        }
    return;
  }
  if constexpr (OUT_F32 && !SWIGLU) {
    // fp32 output: every store already writes whole 128-byte row pieces
    // (32 lanes x 4 bytes), so no staging; measured against the staged
    // path: DeepSeek-shape down 2.01 -> 1.97 ms, Mixtral-shape 0.94 -> 0.93.
    // An output larger than the last-level cache streams to HBM anyway and
    // is stored non-temporally (DeepSeek shapes, 1.06 GB: down 1880 ->
    // 1823 us, the combine that reads it 229 -> 221 us; an output that fits,
    // as on the Mixtral shapes, stays cached for the combine)
    float *const cb = static_cast<float *>(C) + (size_t)tile.nt * BN + col;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = tile.m0 + wm * (MI * 32) + mi * 32 + 8 * (r >> 2) + rbase + (r & 3);
        if (m < tile.mend) {
          float *const rp = cb + (size_t)m * N;
          if (nt_store) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              __builtin_nontemporal_store(acc[mi][nb][r], &rp[b_row<SWIGLU, NWN>(wn, nb)]);
          } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) rp[b_row<SWIGLU, NWN>(wn, nb)] = acc[mi][nb][r];
          }
        }
      }
    return;
  }
  if constexpr (SWIGLU && !OUT_F32) {
    // bf16 gate/up output: the whole tile (BM rows x 128 columns, at most
    // 64 KB) is staged at once -- wave row wm into A slot wm, both free once
    // every wave is past the last stage -- then every thread stores its
    // 16-byte row pieces: one barrier instead of two per 32-row block, all
    // of a thread's stores in flight together.  The 16-byte piece index is
    // XORed with bit 2 of the row, so the two rows one write instruction
    // touches (4 apart) fall in different banks.
    constexpr int TC = BN / 2;      // output columns of the tile
    constexpr int ROWB = TC * 2;    // bytes per staged row
    constexpr int PPR = ROWB / 16;  // 16-byte pieces per row
    constexpr int WR = MI * 32;     // rows of one wave row
    static_assert(WR * ROWB <= (int)sizeof(u32x4) * SLOTS_A2MAX, "a wave row must fit an A slot");
    __syncthreads();  // every wave is done reading the rings
    char *const stg_w = reinterpret_cast<char *>(wm == 0 ? sA0 : sA1);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int nb = 0; nb < NB / 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mi * 32 + 8 * (r >> 2) + rbase + (r & 3);
          const int c = wn * (TC / NWN) + nb * 32 + col;
          const float g = acc[mi][nb][r], u = acc[mi][nb + NB / 2][r];
          // hardware exp2 and reciprocal (each within 1 ulp; far below the
          // bf16 rounding)
          const float v = g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * g)) * u;
          const int off = row * ROWB + ((((c * 2) >> 4) ^ ((row >> 2) & 1)) << 4) + ((c * 2) & 15);
          *reinterpret_cast<__bf16 *>(stg_w + off) = (__bf16)v;  // round to nearest even
        }
    __syncthreads();
    const size_t col0 = (size_t)tile.nt * TC;
#pragma unroll
    for (int i = 0; i < (2 * WR * PPR) / (NW * 64); ++i) {
      const int q = i * (NW * 64) + tid;
      const int wr = q / (WR * PPR), rr = (q / PPR) % WR, pc = q % PPR;
      const int m = tile.m0 + wr * WR + rr;
      if (m < tile.mend) {
        const char *sp = reinterpret_cast<const char *>(wr == 0 ? sA0 : sA1) + rr * ROWB +
                         ((pc ^ ((rr >> 2) & 1)) << 4);
        *reinterpret_cast<u32x4 *>(static_cast<char *>(C) + ((size_t)m * N + col0) * 2 + pc * 16) =
            *reinterpret_cast<const u32x4 *>(sp);
      }
    }
    return;
  }
  // Output, one 32-row block (mi) of every wave at a time: each wave writes
  // its values into LDS -- wave row wm into B slot wm, free once every wave
  // is past the last stage -- as [32 rows][TC columns] of the output type,
  // then all threads store whole 16-byte row pieces (instead of one 2- or
  // 4-byte store per accumulator element).  The 16-byte piece index is
  // XORed with bit 2 of the row, so the two rows one write instruction
  // touches (4 apart) fall in different banks.
  constexpr int TC = SWIGLU ? BN / 2 : BN;  // output columns of the tile
  constexpr int OSZ = OUT_F32 ? 4 : 2;      // bytes per output element
  constexpr int ROWB = TC * OSZ;            // bytes per staged row
  constexpr int PPR = ROWB / 16;            // 16-byte pieces per row
  static_assert(32 * ROWB <= (int)sizeof(u32x4) * SLOTS_B2, "staging block must fit a B slot");
  __syncthreads();  // every wave is done reading the rings
  char *const stg_w = reinterpret_cast<char *>(wm == 0 ? sB0 : sB1);
  const size_t col0 = (size_t)tile.nt * TC;  // first output column of the tile
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    constexpr int NO = SWIGLU ? NB / 2 : NB;  // 32-column output blocks per wave
#pragma unroll
    for (int nb = 0; nb < NO; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + rbase + (r & 3);
        const int c = wn * (TC / NWN) + nb * 32 + col;
        float v;
        if (SWIGLU) {
          const float g = acc[mi][nb][r], u = acc[mi][nb + NO][r];
          // bf16 output: hardware exp2 and reciprocal (each within 1 ulp;
          // far below the bf16 rounding); fp32 output keeps expf and the
          // IEEE divide
          v = OUT_F32 ? g / (1.0f + expf(-g)) * u
                      : g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * g)) * u;
        } else {
          v = acc[mi][nb][r];
        }
        const int off = row * ROWB + ((((c * OSZ) >> 4) ^ ((row >> 2) & 1)) << 4) + ((c * OSZ) & 15);
        if (OUT_F32)
          *reinterpret_cast<float *>(stg_w + off) = v;
        else
          *reinterpret_cast<__bf16 *>(stg_w + off) = (__bf16)v;  // round to nearest even
      }
    __syncthreads();
    for (int q = tid; q < 2 * 32 * PPR; q += NW * 64) {
      const int wr = q / (32 * PPR), rr = (q / PPR) % 32, pc = q % PPR;
      const int m = tile.m0 + wr * (MI * 32) + mi * 32 + rr;
      if (m < tile.mend) {
        const char *src = reinterpret_cast<const char *>(wr == 0 ? sB0 : sB1) + rr * ROWB +
                          ((pc ^ ((rr >> 2) & 1)) << 4);
        *reinterpret_cast<u32x4 *>(static_cast<char *>(C) + ((size_t)m * N + col0) * OSZ + pc * 16) =
            *reinterpret_cast<const u32x4 *>(src);
      }
    }
    __syncthreads();  // the staging block is rewritten for the next mi
  }
}

// One launch over all groups.  Groups are cut into 256-row tiles; the
// last, partial tile of a group runs with the smallest height in
// {64, 128, 256} that holds its rows, chosen here from the device offsets,
// so a group of 40 rows (or the 40-row tail of a 1064-row group) costs a
// quarter of the matrix-core work and 5/8 of the operand traffic of a full
// tile.  With a workspace, the last n_split tiles (the partial last round)
// are taken by S workgroups each, one K-slice apiece.
template <bool SWIGLU, bool OUT_F32, int NW>
__global__ __launch_bounds__(NW * 64, 1) void gemm_bf16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const uint16_t *__restrict__ B2, void *__restrict__ C, const int32_t *__restrict__ offsets,
    int G, int rows, int N, int K, int ldb, int nt_count, char *__restrict__ ws, int cus,
    int xcd_run, int nt_store) {
  // 2 A double stages (64 KB) and 3 B double stages (96 KB): all 160 KB of LDS.
  // The scheduler's result (8 ints) passes through the last B slot, which is
  // first loaded after every wave has passed the prologue barrier.
  __shared__ u32x4 sA0[SLOTS_A2MAX], sA1[SLOTS_A2MAX];
  __shared__ u32x4 sB0[SLOTS_B2], sB1[SLOTS_B2], sB2[SLOTS_B2];
  const int KT = K / BK;  // a multiple of 4
  const int w = (int)blockIdx.x;
  // workgroups [0, full_end) take one tile each; with a split tail, S
  // workgroups per tile after that, one K-slice each
  auto plan = [&](int total, int *S, int *n_split, int *full_end) {
    *S = ws != nullptr ? split_slices(total, cus, KT) : 1;
    *n_split = *S > 1 ? total % cus : 0;
    *full_end = total - *n_split;
  };
  auto pick = [&](int total) {
    int S, n_split, full_end;
    plan(total, &S, &n_split, &full_end);
    if (w < full_end) {
      // XCD-local order: in every whole block of 8 xcd_run workgroups, XCD x
      // (the workgroups w = x mod 8) takes xcd_run consecutive tile ids
      if (xcd_run <= 0) return w;
      const int span = 8 * xcd_run, blk = w / span;
      if ((blk + 1) * span > full_end) return w;
      const int i = w - blk * span;
      return blk * span + (i % 8) * xcd_run + i / 8;
    }
    const int jj = (w - full_end) / S;
    return jj < n_split ? full_end + jj : -1;
  };
  // the scheduler's result lives in the last B slot until the prologue
  const Sched sc = sched_lookup(offsets, G, rows, BM_MAX, nt_count, kTileChunk, SWIGLU,
                                reinterpret_cast<int *>(sB2), pick);
  int S, n_split, full_end;
  plan(sc.total, &S, &n_split, &full_end);
  if (ws != nullptr && w == 0 && threadIdx.x == 0) {
    int *hdr = reinterpret_cast<int *>(ws);
    hdr[0] = n_split;
    hdr[1] = S;
  }
  if (sc.L < 0) return;
  int kbeg = 0, kt = KT, j = -1, slice = 0;
  float *part = nullptr;
  if (w >= full_end) {  // a K-slice of split tile j
    j = (w - full_end) / S;
    slice = (w - full_end) - j * S;
    kt = KT / S;
    kbeg = slice * kt * BK;
    part = reinterpret_cast<float *>(ws + split_partial_offset(cus)) +
           (size_t)(j * S + slice) * kPartialFloats;
  }
  const Tile tile = sc.tile;
  if (part != nullptr && slice == 0 && threadIdx.x == 0)
    reinterpret_cast<int4 *>(ws + split_desc_offset())[j] = make_int4(tile.m0, tile.mend, tile.nt, 0);
  const int h = tile.mend - tile.m0;  // wave-uniform
  // SwiGLU (gate/up) tiles with at least one dead 32-row block skip it;
  // measured: DeepSeek-shape gate/up 3.53 -> 3.41 ms, no change on the
  // Mixtral shapes.  Down-projection tiles never skip: the extra control
  // flow cost more than the saved MFMAs there.
#define MOE_TILE(BMV, SKIPV)                                                                  \
  run_tile<BMV, SWIGLU, OUT_F32, NW, SKIPV>(tile, A, B, B2, C, rows, N, K, ldb, kbeg, kt, part, sA0, \
                                            sA1, sB0, sB1, sB2, nt_store != 0)
  if (h > 128) {
    if (SWIGLU && h <= 224) MOE_TILE(256, SWIGLU); else MOE_TILE(256, false);
  } else if (h > 64) {
    if (SWIGLU && h <= 96) MOE_TILE(128, SWIGLU); else MOE_TILE(128, false);
  } else {
    if (SWIGLU && h <= 32) MOE_TILE(64, SWIGLU); else MOE_TILE(64, false);
  }
#undef MOE_TILE
}

// Sum of the S partial tiles of each split tile, in slice order, then the
// epilogue.  Work item (j, rb) is rows [16 rb, 16 rb + 16) of split tile j;
// items run row block by row block across the split tiles (item = rb *
// n_split + j), so the live blocks of short tiles are all taken in the
// grid's first pass (decode-size layer: down 190 -> 180 us, gate/up 337 ->
// 331 us, against tile by tile); the grid is four workgroups per CU looping
// over the items, so the launch stays cheap when nothing was split (the
// plan is only known on the device).  A thread owns RPT (row, 4-column
// group) pairs of an item and issues the loads of all of them, every slice,
// before the first add (16 bytes per partial); the adds then run in slice
// order.
constexpr int kReduceRows = 16;
constexpr int kReduceWGPerCU = 4;

template <bool SWIGLU, bool OUT_F32>
__global__ __launch_bounds__(256) void split_reduce_kernel(const char *__restrict__ ws,
                                                           void *__restrict__ C, int N, int cus) {
  const int *hdr = reinterpret_cast<const int *>(ws);
  const int n_split = hdr[0], S = hdr[1];
  constexpr int RB = BM_MAX / kReduceRows;
  constexpr int C4 = SWIGLU ? BN / 8 : BN / 4;  // 4-column groups per output row
  constexpr int RPT = kReduceRows * C4 / 256;   // (row, group) pairs per thread
  static_assert(RPT * 256 == kReduceRows * C4, "an item is a whole number of passes");
  for (int item = blockIdx.x; item < n_split * RB; item += gridDim.x) {
    const int j = item % n_split, r0 = (item / n_split) * kReduceRows;
    const int4 d = reinterpret_cast<const int4 *>(ws + split_desc_offset())[j];
    const int h = d.y - d.x;
    if (r0 >= h) continue;
    const float *P = reinterpret_cast<const float *>(ws + split_partial_offset(cus)) +
                     (size_t)j * S * kPartialFloats;
    float4 g[RPT][kSplitMax], u[RPT][kSplitMax];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int idx = i * 256 + (int)threadIdx.x;
      const int r = r0 + idx / C4, c = (idx % C4) * 4;
      const float *p0 = P + (size_t)r * BN + c;
#pragma unroll
      for (int q = 0; q < kSplitMax; ++q) {
        if (q < S && r < h) {
          g[i][q] = *reinterpret_cast<const float4 *>(p0 + q * kPartialFloats);
          if (SWIGLU) u[i][q] = *reinterpret_cast<const float4 *>(p0 + q * kPartialFloats + BN / 2);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int idx = i * 256 + (int)threadIdx.x;
      const int r = r0 + idx / C4, c = (idx % C4) * 4;
      if (r >= h) continue;
      float4 gs = g[i][0], us = SWIGLU ? u[i][0] : float4{};
#pragma unroll
      for (int q = 1; q < kSplitMax; ++q) {
        if (q < S) {
          gs.x += g[i][q].x; gs.y += g[i][q].y; gs.z += g[i][q].z; gs.w += g[i][q].w;
          if (SWIGLU) { us.x += u[i][q].x; us.y += u[i][q].y; us.z += u[i][q].z; us.w += u[i][q].w; }
        }
      }
      float v[4] = {gs.x, gs.y, gs.z, gs.w};
      if (SWIGLU) {
        const float uu[4] = {us.x, us.y, us.z, us.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)  // silu as in the tile epilogue
          v[e] = OUT_F32 ? v[e] / (1.0f + expf(-v[e])) * uu[e]
                         : v[e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * v[e])) * uu[e];
      }
      const size_t o = (size_t)(d.x + r) * N + (size_t)d.z * (SWIGLU ? BN / 2 : BN) + c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (OUT_F32) static_cast<float *>(C)[o + e] = v[e];
        else static_cast<uint16_t *>(C)[o + e] = f32_to_bf16_bits(v[e]);
      }
    }
  }
}

template <bool SWIGLU, bool OUT_F32, int NW>
void launch_t(const void *A, const void *B, const void *B2, void *C, const int32_t *offsets,
              int G, int rows, int N, int K, int ldb, char *ws, int cus, hipStream_t s) {
  const int nt = SWIGLU ? N / 128 : N / 256;
  // slices of split tiles add at most cus - 1 workgroups past the tile count
  const long long bound = (long long)host_row_tile_bound(rows, G, BM_MAX) * nt + (ws ? cus : 0);
  // SwiGLU over groups of at most one 256-row tile on average (fine-grained
  // experts): each expert's column tiles go to one XCD, so its rows are
  // fetched into one L2 rather than eight (DeepSeek shapes, one process:
  // gate/up 3139 -> 3099 us; the down projection was slower that way, 1906 ->
  // 2011 us, and keeps the default order)
  const int xcd_run = (SWIGLU && (long long)rows <= 256LL * G) ? nt : 0;
  const int nt_store = (OUT_F32 && !SWIGLU && (long long)rows * N * 4 > kLastLevelCacheBytes) ? 1 : 0;
  hipLaunchKernelGGL((gemm_bf16_kernel<SWIGLU, OUT_F32, NW>), dim3((unsigned)((bound + 7) / 8 * 8)),
                     dim3(NW * 64), 0, s, static_cast<const uint16_t *>(A),
                     static_cast<const uint16_t *>(B), static_cast<const uint16_t *>(B2), C,
                     offsets, G, rows, N, K, ldb, nt, ws, cus, xcd_run, nt_store);
  if (ws == nullptr) return;
  hipLaunchKernelGGL((split_reduce_kernel<SWIGLU, OUT_F32>), dim3((unsigned)(kReduceWGPerCU * cus)),
                     dim3(256), 0, s,
                     ws, C, N, cus);
}

}  // namespace

bool gemm_bf16_mfma_supports(int N, int K, int epi) {
  if (K <= 0 || K % (4 * BK) != 0) return false;
  return epi == MOE_EPI_SWIGLU ? (N % 128 == 0) : (N % 256 == 0);
}

size_t gemm_bf16_split_ws_bytes(int G, int rows, int N, int K, int epi, int cus) {
  if (!gemm_bf16_mfma_supports(N, K, epi) || cus < 2) return 0;
  const int KT = K / BK;
  int smax = kSplitMax;
  while (smax > 1 && (KT % (4 * smax) != 0 || KT / smax < kSplitMinSteps)) smax >>= 1;
  if (smax < 2) return 0;
  const int nt = epi == MOE_EPI_SWIGLU ? N / 128 : N / 256;
  const long long tiles = (long long)host_row_tile_bound(rows, G, BM_MAX) * nt;
  const long long slices = tiles * smax < cus ? tiles * smax : cus;  // n_split * S <= both
  return split_partial_offset(cus) + (size_t)slices * kPartialFloats * sizeof(float);
}

hipError_t launch_gemm_bf16_mfma(const void *A, const void *B, const void *B2, void *C, int c_dt,
                                 const int32_t *offsets, int G, int rows, int N, int K, int ldb,
                                 int epi, void *ws, int cus, hipStream_t s) {
  char *w = static_cast<char *>(ws);
  // wave counts measured on the Mixtral shapes: 8 for gate/up, 4 for down
  if (epi == MOE_EPI_SWIGLU) {
    if (c_dt == MOE_F32) launch_t<true, true, 8>(A, B, B2, C, offsets, G, rows, N, K, ldb, w, cus, s);
    else launch_t<true, false, 8>(A, B, B2, C, offsets, G, rows, N, K, ldb, w, cus, s);
  } else {
    if (c_dt == MOE_F32) launch_t<false, true, 4>(A, B, B2, C, offsets, G, rows, N, K, ldb, w, cus, s);
    else launch_t<false, false, 4>(A, B, B2, C, offsets, G, rows, N, K, ldb, w, cus, s);
  }
  return hipGetLastError();
}

