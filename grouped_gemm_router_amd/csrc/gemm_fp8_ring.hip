// gemm_fp8_ring.hip -- FP8 (E4M3) block-scaled grouped GEMM for gfx950,
// operands streamed through LDS rings of LDS-direct loads.
//
// "DeepGEMM walkthrough" §2.3 (C ~ (A_q / scale_A)(B_q / scale_B); the
// stored scales here are the dequantisation multipliers, the reciprocal of
// the page's scale), §5.1 (scales per token group and per weight block woven
// into the GEMM, fp32 accumulation), §4.3 (one launch over ragged groups),
// §5.2 (multi-buffered loads), §5.3 (masked tails).
//   C[r][n] = sum_kb sA[r][kb] * sB[g][n/128][kb] * (sum_{k in kb} Aq Bq)
//
// Design (CDNA4, 64-wide waves, 8 waves in a 2 x 4 grid):
//   * a K step is 64 fp8 columns; operand rows move HBM/L2 -> LDS with
//     global_load_lds_dwordx4 as whole 128-byte pieces, i.e. two steps = one
//     128-column scale block at a time (the TCP sends one L2 request per
//     line touched: half the requests of 64-byte pieces).  A runs through
//     two such double-step slots, B through three, refilled one and two
//     double steps ahead; each double step waits only for its own loads and
//     meets the other waves at one plain s_barrier.  Measured on the
//     DeepSeek shapes against 4-stage rings of 64-byte pieces: gate/up 2.03
//     -> 1.90 ms, down 1.11 -> 1.04 ms;
//   * one v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit E8M0 block
//     scales) per 32 x 32 block and step; its result is the exact-scale
//     partial sum of 64 products, folded into the fp32 accumulator with the
//     fp32 factor sA * sB of its 128-column scale block (two steps share a
//     block): the promotion to fp32 happens every 64 columns;
//   * the weight tile is the MFMA's row operand and the token tile its column
//     operand, so a lane holds one token: the fold needs one sA per lane and
//     one sB per wave column (a scalar load), not one per accumulator row;
//   * activation scales are stored group-major, [K/128][rows], so one
//     block's scales for the tile rows are one contiguous run; they travel
//     with their block's A double step: one 4-byte LDS-direct load per wave
//     (32 rows, each fetched by two lanes) into the scale slot of that A
//     slot, read once per block;
//   * tile heights 64 / 128 / 192 rows are chosen per tile from its row
//     count, as in the bf16 kernel (a group's last tile shrinks to what it
//     holds); 192, not 256: two 256-row A slots, three B slots and the scale
//     slots do not fit the 160 KB of LDS;
//   * the main loop runs six double steps per trip (the slot pattern
//     repeats every six); the K % 768 / 128 double steps that do not fill a
//     trip run ahead of it, and the loop then starts at that phase of the
//     pattern, so its body has no exit.  Exits inside the body made the
//     compiler drain every load once per trip (4-5 %), a tail after the
//     loop spilled the accumulators;
//   * SwiGLU: the weight tile holds 128 gate rows then the 128 matching up
//     rows; wave column wn takes gate rows [32 wn, +32) and up rows
//     [128 + 32 wn, +32), so silu(gate) * up pairs in registers; E4M3 output
//     quantises each row's 128 h columns of the tile as one 1 x 128 group
//     (absmax over the lane pair, then over the four wave columns in LDS).
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int BM_MAX = 192, BN = 256, BK = 64;  // BK: fp8 columns (= bytes) per step
constexpr int PIECES = BK / 16;                 // 16-byte pieces per tile row (4)
constexpr int PIECES2 = 2 * PIECES;             // 16-byte pieces per 128-byte row (two steps)
constexpr int SLOTS_A2MAX = BM_MAX * PIECES2;   // 16-byte slots per A double step (24 KB)
constexpr int SLOTS_B2 = BN * PIECES2;          // 16-byte slots per B double step (32 KB)
constexpr int NW = 8, NWN = 4;                  // waves, wave columns (2 wave rows)
constexpr int NB = 2;                           // 32-row weight blocks per wave
constexpr int NTH = NW * 64;
constexpr int SROWS = NW * 64;                  // activation-scale slot (32 rows per wave, x2)

// piece p of a 128-byte row r sits at slot p ^ ((r >> 1) & 7) of the row
__device__ __forceinline__ int swz(int row, int p) { return p ^ ((row >> 1) & 7); }

// weight-tile row of wave column wn, 32-row block nb
template <bool SWIGLU>
__device__ __forceinline__ int b_row(int wn, int nb) {
  return SWIGLU ? nb * 128 + wn * 32 : wn * 64 + nb * 32;
}

// Output conversions of the epilogues.  silu uses the hardware exp2 and
// reciprocal (each within 1 ulp), far below the bf16 / E4M3 rounding that
// follows; E4M3 codes come from e4m3x4 (the per-row scale keeps the values
// in [-448, 448]); bf16 from the hardware round-to-nearest-even conversion.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * g)) * u;
}
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

template <int SZ>
__device__ __forceinline__ void dma_to_lds(const void *g, void *l) {
  if constexpr (SZ == 16)
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 4, 0, 0);
}

// the 32 bytes (64 K columns split in two lane halves) of row r in step
// `par` (0 or 1) of a double step
__device__ __forceinline__ i32x8 frag(const u32x4 *t, int r, int fh, int par) {
  const u32x4 lo = t[r * PIECES2 + swz(r, par * PIECES + 2 * fh)];
  const u32x4 hi = t[r * PIECES2 + swz(r, par * PIECES + 2 * fh + 1)];
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

struct Ring {
  u32x4 *a0, *a1;       // A double steps (separate LDS arrays)
  u32x4 *b0, *b1, *b2;  // B double steps
  float *s0, *s1;       // activation scales of A slot 0 / 1's scale block
  float *amax;          // [NWN][BM_MAX], in A slot 0 (epilogue only)
};

template <int BM, bool SWIGLU, bool OUT_FP8, bool SKIP>
__device__ __forceinline__ void run_tile(const Tile &tile, const uint8_t *__restrict__ Aq,
                                         const float *__restrict__ As,
                                         const uint8_t *__restrict__ Bq,
                                         const float *__restrict__ Bs,
                                         const uint8_t *__restrict__ B2q,
                                         const float *__restrict__ B2s, void *__restrict__ C,
                                         float *__restrict__ Cs, int rows, int N, int K,
                                         int ldb, const Ring &ring) {
  constexpr int MI = BM / 64;            // 32-token blocks per wave
  constexpr int SLOTS_A2 = BM * PIECES2;
  constexpr int IA = SLOTS_A2 / NW / 64;  // A loads per wave and double step
  constexpr int IB = SLOTS_B2 / NW / 64;  // B loads per wave and double step
  static_assert(IA >= 1 && IB >= 1, "tile too small for the wave count");

  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  const int wm = wv / NWN, wn = wv % NWN;
  // SKIP (a tile with fewer than BM rows): this wave's 32-row blocks that
  // hold rows of the group; blocks past the group end are neither read nor
  // multiplied nor folded.  Each SIMD runs one wave of each wave row, so the
  // work saved in the mostly empty second wave row shortens the tile.
  int live = MI;
  if (SKIP) {
    const int hv = __builtin_amdgcn_readfirstlane(tile.mend - tile.m0 - wm * (MI * 32));
    live = hv <= 0 ? 0 : min(MI, (hv + 31) / 32);
  }
  const int KB = K / 128, NBK = N / 128;  // scale blocks along K and N

  // LDS-direct sources (whole 128-byte row pieces: two steps, one scale
  // block): wave wv fills slots [wv*SLOTS/NW, +SLOTS/NW) of each double
  // step, 64 per instruction, slot s holding piece swz(row, s % 8) of row
  // s / 8; a wave-uniform base (SGPRs) plus a 32-bit per-lane byte offset
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int gu = __builtin_amdgcn_readfirstlane(tile.g);
  const int ntu = __builtin_amdgcn_readfirstlane(tile.nt);
  uint32_t ga[IA];
  uint32_t gb[IB];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int sl = wv * (SLOTS_A2 / NW) + i * 64 + lane;
    const int r = sl / PIECES2;
    // rows past the tile's last row repeat that row (one address: the loads
    // of dead rows coalesce and hit the L1) and are never stored (DeepSeek
    // shapes: gate/up 1893 -> 1833 us, down 1045 -> 1023 us against
    // clamping to the buffer's last row, which loads the next group's rows)
    const int m = min(tile.m0 + r, tile.mend - 1);
    ga[i] = (uint32_t)m * (uint32_t)K + swz(r, sl % PIECES2) * 16;
  }
  // the B tile of wave wv comes from one matrix: SwiGLU waves 0-3 fill the
  // 128 gate rows, waves 4-7 the 128 up rows
  const uint8_t *bbase = ((SWIGLU && wvu >= NW / 2) ? B2q : Bq) + (size_t)gu * N * ldb;
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    const int sl = wv * (SLOTS_B2 / NW) + i * 64 + lane;
    const int r = sl / PIECES2;
    const int n = SWIGLU ? ntu * 128 + (r & 127)
                         : min(ntu * 256 + r, N - 1);  // N % 256 == 128: half tile
    gb[i] = (uint32_t)n * (uint32_t)ldb + swz(r, sl % PIECES2) * 16;
  }
  // activation scales [K/128][rows]: each A double step carries its block's
  // scales into the matching scale slot; wave wv loads tile rows [32 wv,
  // +32), each by lanes l and l + 32 (the second copy lands in an unused
  // half); rows past the tile read its last row and are never used
  const uint32_t gs = (uint32_t)min(tile.m0 + wv * 32 + (lane & 31), tile.mend - 1) * 4u;
  const int dma_a = wv * (SLOTS_A2 / NW);
  const int dma_b = wv * (SLOTS_B2 / NW);
  float sa[MI];  // this lane's token scales for the current block
  // issue order per double step: A(kb) with its scales, then B(kb + 1)
#define MOE_ISSUE_A(dA, dS, kb)                                                             \
  _Pragma("unroll") for (int i = 0; i < IA; ++i)                                           \
    dma_to_lds<16>(Aq + (ga[i] + (kb) * 128), (dA) + dma_a + i * 64);                      \
  dma_to_lds<4>(reinterpret_cast<const uint8_t *>(As + (size_t)(kb) * rows) + gs, (dS) + wv * 64);
#define MOE_ISSUE_B(dB, kb)                                                                 \
  _Pragma("unroll") for (int i = 0; i < IB; ++i)                                           \
    dma_to_lds<16>(bbase + (gb[i] + (kb) * 128), (dB) + dma_b + i * 64);

  // weight scales of this wave's two 32-row blocks: [g][n-block][kb]; the
  // indices are wave-uniform, so these are scalar loads
  const int wnu = wvu % NWN;
  const float *sb0, *sb1;
  if (SWIGLU) {
    sb0 = Bs + ((size_t)gu * NBK + ntu) * KB;
    sb1 = B2s + ((size_t)gu * NBK + ntu) * KB;
  } else {
    sb0 = Bs + ((size_t)gu * NBK + min(ntu * 2 + wnu / 2, NBK - 1)) * KB;
    sb1 = sb0;
  }

  f32x16 acc[MI][NB];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};
  // tiles of at most 128 rows have the registers to chain the two MFMAs of
  // a 128-column scale block and fold once per block (the fold is VALU work
  // that bounds this kernel); taller tiles fold after every MFMA
  constexpr bool FOLD2 = BM <= 128;
  f32x16 pt[FOLD2 ? MI : 1][NB];
  const int fr = lane & 31, fh = lane >> 5;

  // Double step d (K columns [128 d, 128 d + 128), one scale block): A from
  // slot d % 2, B from slot d % 3.  Loads go out in the order A(d+1),
  // scales(d+1), B(d+2), so waiting until only the last B's IB loads may be
  // outstanding makes A(d), scales(d) and B(d) land; one barrier per double
  // step makes them visible and frees the slots of double step d-1, which
  // take A(d+1) and B(d+2).  The wait also covers the wave's own LDS reads
  // (lgkmcnt 0): the compiler may sink the last multiplies of step d-1 below
  // the barrier, and a read of a step d-1 slot still queued there could
  // otherwise return data of the refill another wave issues right after it.
  // Past the end the last block is re-loaded into slots nobody reads, so the
  // count never changes.
  MOE_ISSUE_A(ring.a0, ring.s0, 0);
  MOE_ISSUE_B(ring.b0, 0);
  MOE_ISSUE_B(ring.b1, min(1, KB - 1));

#define MOE_DSTEP(tA, tS, tB, nA, nS, nB, dd)                                               \
  {                                                                                         \
    wait_vmcnt_lgkm0<IB>();                                                                 \
    stage_barrier();                                                                        \
    _Pragma("unroll") for (int mi = 0; mi < MI; ++mi) {                                     \
      const int r = wm * (MI * 32) + mi * 32 + fr;                                          \
      sa[mi] = (tS)[(r >> 5) * 64 + (r & 31)];                                              \
    }                                                                                       \
    MOE_ISSUE_A(nA, nS, min((dd) + 1, KB - 1));                                             \
    MOE_ISSUE_B(nB, min((dd) + 2, KB - 1));                                                 \
    const int du_ = __builtin_amdgcn_readfirstlane(dd); /* uniform: scalar loads */        \
    const float s0 = sb0[du_], s1 = sb1[du_];                                               \
    _Pragma("unroll") for (int par = 0; par < 2; ++par) {                                   \
      __builtin_amdgcn_sched_barrier(0);                                                    \
      i32x8 w[NB];                                                                          \
      _Pragma("unroll") for (int nb = 0; nb < NB; ++nb)                                     \
        w[nb] = frag(tB, b_row<SWIGLU>(wn, nb) + fr, fh, par);                              \
      _Pragma("unroll") for (int mi = 0; mi < MI; ++mi) {                                   \
        if (mi >= live) break;                                                              \
        const i32x8 x = frag(tA, wm * (MI * 32) + mi * 32 + fr, fh, par);                   \
        _Pragma("unroll") for (int nb = 0; nb < NB; ++nb) {                                 \
          if (FOLD2 && par == 0) {                                                          \
            pt[FOLD2 ? mi : 0][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(       \
                w[nb], x, f32x16{}, 0, 0, 0, 127, 0, 127);                                  \
          } else {                                                                          \
            const f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(               \
                w[nb], x, FOLD2 ? pt[FOLD2 ? mi : 0][nb] : f32x16{}, 0, 0, 0, 127, 0, 127); \
            const float c = sa[mi] * (nb == 0 ? s0 : s1);                                   \
            _Pragma("unroll") for (int r2 = 0; r2 < 16; ++r2)                               \
              acc[mi][nb][r2] = fmaf(p[r2], c, acc[mi][nb][r2]);                            \
          }                                                                                 \
        }                                                                                   \
      }                                                                                     \
    }                                                                                       \
  }
  // the six phases of the slot pattern: (A, its scales, B) read by double
  // step d = 6 t + p, then the slots that take A(d+1) and B(d+2)
#define MOE_P0(dd) MOE_DSTEP(ring.a0, ring.s0, ring.b0, ring.a1, ring.s1, ring.b2, (dd))
#define MOE_P1(dd) MOE_DSTEP(ring.a1, ring.s1, ring.b1, ring.a0, ring.s0, ring.b0, (dd))
#define MOE_P2(dd) MOE_DSTEP(ring.a0, ring.s0, ring.b2, ring.a1, ring.s1, ring.b1, (dd))
#define MOE_P3(dd) MOE_DSTEP(ring.a1, ring.s1, ring.b0, ring.a0, ring.s0, ring.b2, (dd))
#define MOE_P4(dd) MOE_DSTEP(ring.a0, ring.s0, ring.b1, ring.a1, ring.s1, ring.b0, (dd))
#define MOE_P5(dd) MOE_DSTEP(ring.a1, ring.s1, ring.b2, ring.a0, ring.s0, ring.b1, (dd))

  // KB is even.  The first KB % 6 double steps run ahead of the loop, so
  // the loop runs whole trips of six and has no exit in its body (exits
  // there make the compiler drain every load once per trip: 4-5 % measured)
  const int head = KB % 6;
  if (head == 0) {
    for (int kb = 0; kb < KB; kb += 6) {
      MOE_P0(kb) MOE_P1(kb + 1) MOE_P2(kb + 2) MOE_P3(kb + 3) MOE_P4(kb + 4) MOE_P5(kb + 5)
    }
  } else if (head == 2) {
    MOE_P0(0) MOE_P1(1)
    for (int kb = 2; kb < KB; kb += 6) {
      MOE_P2(kb) MOE_P3(kb + 1) MOE_P4(kb + 2) MOE_P5(kb + 3) MOE_P0(kb + 4) MOE_P1(kb + 5)
    }
  } else {
    MOE_P0(0) MOE_P1(1) MOE_P2(2) MOE_P3(3)
    for (int kb = 4; kb < KB; kb += 6) {
      MOE_P4(kb) MOE_P5(kb + 1) MOE_P0(kb + 2) MOE_P1(kb + 3) MOE_P2(kb + 4) MOE_P3(kb + 5)
    }
  }
  wait_vmcnt<0>();  // no LDS-direct load may still be landing when the tile ends
  __syncthreads();  // every wave is past its reads of the slots the epilogue reuses
#undef MOE_P0
#undef MOE_P1
#undef MOE_P2
#undef MOE_P3
#undef MOE_P4
#undef MOE_P5
#undef MOE_DSTEP
#undef MOE_ISSUE_A
#undef MOE_ISSUE_B

  // epilogue.  32x32 accumulator layout: lane holds column (token) lane%32;
  // register r holds row (weight row) 8*(r/4) + 4*(lane/32) + r%4, so each
  // lane holds four runs of four consecutive output columns.
  if (SWIGLU) {
    // h for this lane's tokens: columns nt*128 + 32 wn + 8 j + 4 fh + i
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int ml = wm * (MI * 32) + mi * 32 + fr;
      const int m = tile.m0 + ml;
      float h[16];
      float mx = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        h[r] = silu_mul(acc[mi][0][r], acc[mi][1][r]);
        mx = fmaxf(mx, fabsf(h[r]));
      }
      if (OUT_FP8) {
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        if (fh == 0) ring.amax[wn * BM_MAX + ml] = mx;
      } else if (m < tile.mend) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = tile.nt * 128 + wn * 32 + 8 * j + 4 * fh;
          *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(C) + (size_t)m * N + n) =
              uint2{bf16x2_bits(h[4 * j], h[4 * j + 1]), bf16x2_bits(h[4 * j + 2], h[4 * j + 3])};
        }
      }
      if (OUT_FP8) {
        // every wave reaches this barrier the same number of times (MI is
        // uniform); the four wave columns' maxima of row ml are then visible
        __syncthreads();
        const float amax = fmaxf(fmaxf(ring.amax[ml], ring.amax[BM_MAX + ml]),
                                 fmaxf(ring.amax[2 * BM_MAX + ml], ring.amax[3 * BM_MAX + ml]));
        const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
        const float inv = 1.0f / sc;
        if (m < tile.mend) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = tile.nt * 128 + wn * 32 + 8 * j + 4 * fh;
            *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(C) + (size_t)m * N + n) =
                e4m3x4(h[4 * j] * inv, h[4 * j + 1] * inv, h[4 * j + 2] * inv, h[4 * j + 3] * inv);
          }
          if (wn == 0 && fh == 0) Cs[(size_t)tile.nt * rows + m] = sc;
        }
        __syncthreads();  // the amax slots are rewritten for the next mi
      }
    }
  } else if (!OUT_FP8) {
    // bf16 output, staged whole: every wave writes its 32-token x 64-column
    // blocks into LDS as [32 tokens][256 columns] blocks -- tile row block
    // b = wm * MI + mi in half b % 2 of B slot b / 2 (the whole tile is at
    // most 192 x 256 x 2 bytes, the three B slots) -- then, after one
    // barrier, every thread stores its whole 16-byte row pieces, all in
    // flight together (the direct stores would write 16 bytes into each of 32
    // rows per instruction).  The 16-byte piece index is XORed with the token
    // row, so the reads are conflict free.
    constexpr int BLK = 32 * 512;  // bytes per staged 32-row block
    static_assert(2 * BLK <= (int)sizeof(u32x4) * SLOTS_B2, "two row blocks per B slot");
    static_assert(BM <= 6 * 32, "the tile must fit the three B slots");
    char *const s0 = reinterpret_cast<char *>(ring.b0);
    char *const s1 = reinterpret_cast<char *>(ring.b1);
    char *const s2 = reinterpret_cast<char *>(ring.b2);
    auto slot = [s0, s1, s2](int b) -> char * {
      const int sl = b >> 1;
      return (sl == 0 ? s0 : (sl == 1 ? s1 : s2)) + (b & 1) * BLK;
    };
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      char *const stg = slot(wm * MI + mi);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int pc = wn * 8 + nb * 4 + j;  // 16-byte piece of the staged row
          *reinterpret_cast<uint2 *>(stg + fr * 512 + ((pc ^ fr) << 4) + fh * 8) =
              uint2{bf16x2_bits(acc[mi][nb][4 * j], acc[mi][nb][4 * j + 1]),
                    bf16x2_bits(acc[mi][nb][4 * j + 2], acc[mi][nb][4 * j + 3])};
        }
    }
    __syncthreads();
    static_assert((BM * 32) % NTH == 0, "whole store passes");
#pragma unroll
    for (int i = 0; i < BM * 32 / NTH; ++i) {
      const int q = i * NTH + tid;
      const int row = q >> 5, pc = q & 31, rr = row & 31;
      const int m = tile.m0 + row;
      const int n = tile.nt * 256 + pc * 8;
      if (m < tile.mend && n < N)
        *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(C) + (size_t)m * N + n) =
            *reinterpret_cast<const u32x4 *>(slot(row >> 5) + rr * 512 + ((pc ^ rr) << 4));
    }
  } else {
    // columns nt*256 + 64 wn + 32 nb + 8 j + 4 fh + i; quantisation group
    // (E4M3 output) = wave columns {0,1} and {2,3}
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int ml = wm * (MI * 32) + mi * 32 + fr;
      const int m = tile.m0 + ml;
      const int nbase = tile.nt * 256 + wn * 64;
      const bool live = nbase < N && m < tile.mend;
      float sc = 1.0f;
      if (OUT_FP8) {
        float mx = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(acc[mi][nb][r]));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        if (fh == 0) ring.amax[wn * BM_MAX + ml] = mx;
        __syncthreads();
        const int w0 = wn & ~1;
        const float amax = fmaxf(ring.amax[w0 * BM_MAX + ml], ring.amax[(w0 + 1) * BM_MAX + ml]);
        sc = amax > 0.f ? amax / 448.0f : 1.0f;
        __syncthreads();
      }
      if (!live) continue;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = nbase + nb * 32 + 8 * j + 4 * fh;
          const float v[4] = {acc[mi][nb][4 * j], acc[mi][nb][4 * j + 1],
                              acc[mi][nb][4 * j + 2], acc[mi][nb][4 * j + 3]};
          if (OUT_FP8) {
            const float inv = 1.0f / sc;
            *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(C) + (size_t)m * N + n) =
                e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
          } else {
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(C) + (size_t)m * N + n) =
                uint2{bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
          }
        }
      if (OUT_FP8 && wn % 2 == 0 && fh == 0) Cs[(size_t)(tile.nt * 2 + wn / 2) * rows + m] = sc;
    }
  }
}

template <bool SWIGLU, bool OUT_FP8>
__global__ __launch_bounds__(NTH, 1) void gemm_fp8_ring_kernel(
    const uint8_t *__restrict__ Aq, const float *__restrict__ As, const uint8_t *__restrict__ Bq,
    const float *__restrict__ Bs, const uint8_t *__restrict__ B2q,
    const float *__restrict__ B2s, void *__restrict__ C, float *__restrict__ Cs,
    const int32_t *__restrict__ offsets, int G, int rows, int N, int K, int ldb, int nt_count) {
  // 2 A and 3 B double steps and two scale slots (148 KB of LDS).  The
  // scheduler's result (8 ints) passes through B slot 2, first loaded after
  // every wave has passed the first barrier; the epilogue's row maxima live
  // in A slot 0 once the loop is done.
  __shared__ u32x4 sA0[SLOTS_A2MAX], sA1[SLOTS_A2MAX];
  __shared__ u32x4 sB0[SLOTS_B2], sB1[SLOTS_B2], sB2[SLOTS_B2];
  __shared__ float sS0[SROWS], sS1[SROWS];
  static_assert(sizeof(float) * NWN * BM_MAX <= sizeof(u32x4) * SLOTS_A2MAX,
                "row maxima must fit in one A slot");
  // the scheduler's result lives in the last B slot until the prologue
  const int w = (int)blockIdx.x;
  const Sched sc = sched_lookup(offsets, G, rows, BM_MAX, nt_count, kTileChunk, SWIGLU,
                                reinterpret_cast<int *>(sB2),
                                [w](int total) { return tile_of_workgroup(w, total); });
  if (sc.L < 0) return;
  const Tile tile = sc.tile;
  const Ring ring{sA0, sA1, sB0, sB1, sB2, sS0, sS1, reinterpret_cast<float *>(sA0)};
  const int h = tile.mend - tile.m0;  // wave-uniform
  if (h == BM_MAX)
    run_tile<BM_MAX, SWIGLU, OUT_FP8, false>(tile, Aq, As, Bq, Bs, B2q, B2s, C, Cs, rows, N, K, ldb, ring);
  else if (h > 128)
    run_tile<BM_MAX, SWIGLU, OUT_FP8, true>(tile, Aq, As, Bq, Bs, B2q, B2s, C, Cs, rows, N, K, ldb, ring);
  else if (h > 64)
    run_tile<128, SWIGLU, OUT_FP8, true>(tile, Aq, As, Bq, Bs, B2q, B2s, C, Cs, rows, N, K, ldb, ring);
  else
    run_tile<64, SWIGLU, OUT_FP8, true>(tile, Aq, As, Bq, Bs, B2q, B2s, C, Cs, rows, N, K, ldb, ring);
}

}  // namespace

bool gemm_fp8_ring_supports(int rows, int N, int K, int ldb) {
  // per-lane source offsets are 32-bit: rows x K bytes of A and N x ldb bytes
  // of one group's weights must stay below 4 GiB
  return K > 0 && K % (4 * BK) == 0 && N % 128 == 0 && (long long)rows * K < (1ll << 32) &&
         (long long)N * ldb < (1ll << 32);
}

hipError_t launch_gemm_fp8_ring(const uint8_t *Aq, const float *As, const uint8_t *Bq,
                                const float *Bs, const uint8_t *B2q, const float *B2s, void *C,
                                int c_dt, float *C_scale, const int32_t *offsets, int G,
                                int rows, int N, int K, int ldb, int epi, hipStream_t s) {
  const bool swiglu = epi == MOE_EPI_SWIGLU;
  const int nt = swiglu ? N / 128 : (N + 255) / 256;
  const long long bound = (long long)host_row_tile_bound(rows, G, BM_MAX) * nt;
  const dim3 grid((unsigned)((bound + 7) / 8 * 8)), block(NTH);
  const bool f8 = c_dt == MOE_E4M3;
  if (swiglu) {
    if (f8)
      hipLaunchKernelGGL((gemm_fp8_ring_kernel<true, true>), grid, block, 0, s, Aq, As, Bq, Bs,
                         B2q, B2s, C, C_scale, offsets, G, rows, N, K, ldb, nt);
    else
      hipLaunchKernelGGL((gemm_fp8_ring_kernel<true, false>), grid, block, 0, s, Aq, As, Bq, Bs,
                         B2q, B2s, C, C_scale, offsets, G, rows, N, K, ldb, nt);
  } else {
    if (f8)
      hipLaunchKernelGGL((gemm_fp8_ring_kernel<false, true>), grid, block, 0, s, Aq, As, Bq, Bs,
                         B2q, B2s, C, C_scale, offsets, G, rows, N, K, ldb, nt);
    else
      hipLaunchKernelGGL((gemm_fp8_ring_kernel<false, false>), grid, block, 0, s, Aq, As, Bq, Bs,
                         B2q, B2s, C, C_scale, offsets, G, rows, N, K, ldb, nt);
  }
  return hipGetLastError();
}
