// Expert FFN on the matrix cores: grouped bf16 GEMMs for many rows per expert.
//
// n4n.ai page "How does Grok-1 use a mixture-of-experts design?", section
// "Expert implementation: SwiGLU at scale": an expert is
// w_down(silu(w_gate x) * w_up x), and gate and up can be fused into one
// product over the shared input (FusedSwiGLUExpert). Kernel 1 computes, for
// each expert, the gate and up tiles of the same output columns in one
// work-group and writes h = silu(g) * u (bf16) from the accumulators; kernel 2
// is the down projection y = h W_down^T.
//
// Both operands are k-contiguous (activation rows [m][k], nn.Linear weights
// [n][k]), so each 16-byte load holds 8 consecutive k of one row, which is the
// per-lane operand of v_mfma_f32_32x32x16_bf16.
//
// A work-group of 8 waves computes a tile of activation rows x weight rows,
// of one of two shapes chosen per expert by its row count (from the dispatch
// offsets, on the device): the wide tiles, 256 rows x 256 weight rows (gate
// 128 + up 128, or 256 down columns), waves in a 4 x 2 grid, for experts with
// more than 128 rows; the stream tiles, 128 rows x 512 weight rows, waves in
// a 2 x 4 grid, for experts with at most 128 rows (medium batches), whose
// weights stream once from HBM while the few activation rows are re-read from
// L2 per column tile, so a wider tile means fewer re-reads. Either way each
// wave holds 8 MFMA accumulators of 32x32 (two waves per SIMD). k advances in
// slices of 64 through a two-stage LDS ring filled by direct global->LDS
// loads (global_load_lds_dwordx4, no register staging); the activation rows
// of the gate/up product are gathered from x through the dispatch permutation
// by the addresses of those loads. Each wave loads its MFMA operands for the
// next 16-k step while the current step's MFMAs run, across the stage
// boundary as well, and the scheduler is asked to issue one LDS read after
// each MFMA. LDS rows use a 16-byte-chunk XOR swizzle so the 32 lanes reading
// one chunk column of 32 consecutive rows hit distinct banks.
//
// int8 weights travel to LDS as int8 (half the bytes of the B tile) and are
// converted exactly to bf16 when each wave loads its MFMA operands; their
// per-row scales multiply the float32 accumulators in the epilogue.
#include "common.h"
#include "grouped.h"
#include "kernels.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// direct-to-LDS pipelined grouped GEMM
// ---------------------------------------------------------------------------
constexpr int MBM = 256;   // activation rows per tile
constexpr int MNB = 256;   // weight rows per tile of the wide tiles (the stream tiles: 128)
constexpr int MBK = 64;    // k per LDS stage
constexpr int MNW = 8;                             // waves per work-group
constexpr int MLPW = MBM * 8 / 64 / MNW;           // A LDS-DMA loads per wave per stage
// wave grid (rows x weight rows): 4 x 2 on the wide bf16 tiles; 2 x 4 on the
// stream tiles (128 rows) and with int8 weights, where each converted int8
// operand is then shared by fewer waves (the conversion runs on the VALU once
// per wave that uses the operand)
template <int WT, int BM, int BN> struct WaveGrid {
  static constexpr int M = BM == 256 && !(WT == WT_I8) ? 4 : 2;
  static constexpr int N = MNW / M;
};

typedef __attribute__((address_space(3))) void lds_void_t;

MOE_DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void_t*)p; }

// A wave-uniform pointer, held in scalar registers.
MOE_DEV const char* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// 64 lanes x 16 bytes from global memory into LDS at byte address lds +
// 16*lane (lds wave-uniform), written as asm because the compiler's
// wait-count pass, unable to tell the two LDS stages apart, otherwise drains
// every outstanding load before each LDS read; this kernel places its own
// vmcnt waits. The load writes no VGPR. Two address forms: a scalar base plus
// a per-lane 32-bit byte offset (below 2^31), or a per-lane 64-bit address.
// m0 is named as clobbered on purpose: the asm sets it, and the compiler
// keeps nothing in m0 in these kernels (checked in the generated code).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
MOE_DEV void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
MOE_DEV void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) leaving the other counters untouched
template <int N>
MOE_DEV void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
MOE_DEV void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// work-group barrier that the compiler may not move memory operations across
MOE_DEV void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Modes of ffn_mfma_kernel. M_GATEUP_SAVE is M_GATEUP that also stores the
// pre-activations g and u (bf16), which the backward reads.
enum Mode { M_DOWN = 0, M_GATEUP = 1, M_GATEUP_SAVE = 2 };

template <int WT, int BN> struct BTile {
  static constexpr int ESZ = WT == WT_I8 ? 1 : 2;       // weight element bytes
  static constexpr int BCH = MBK * ESZ / 16;            // 16-byte chunks per B row
  static constexpr int LPW = BN * BCH / 64 / MNW;       // B LDS-DMA loads per wave per stage
};

// s_waitcnt until this wave's loads of the stage being waited for have
// landed while those of `later` (0 .. 2) later stages may still be in flight
// (LPS loads per stage).
template <int LPS>
MOE_DEV void wait_landed(int later) {
  if (later >= 2) wait_vmcnt<2 * LPS>();
  else if (later == 1) wait_vmcnt<LPS>();
  else wait_vmcnt<0>();
}

// The pipelined k loop, shared by the kernels of this file as macros over
// the kernel's own locals (a device function here changed the forward
// kernel's instruction schedule): KT >= 1 stages of MBK through an LDS ring
// of NST stages (NST = 2 or 3; stage s at LDS address Ls[s], the A tile of
// TBM rows then the B tile; SA / SB point at them), NST - 1 stages in flight
// while one is computed. This wave's TLPW A loads read MOE_AADDR(k0) +
// aoff[j] (aptr[j] + 2 k0 when WIDE), its LPWB B loads MOE_BADDR(k0) +
// boff[j]; MOE_LOADA / MOE_LOADB read
// one 16-k step of MFMA operands from a stage into fa / fb (MOE_LOADA for the
// first MIA row blocks); MOE_PRE_MFMA may edit them before the step's MFMAs;
// the scheduler is asked to place MOE_READS_AFTER(q, MIA) LDS reads of the
// next step after the step's q-th MFMA. MIA <= MI row blocks of 32 take part
// (a tile whose rows fit the first MIA blocks skips the others' MFMAs).
// Every kernel defines these hooks before it expands MOE_PIPELINE.
#define MOE_ISSUE(ST, K0)                                                               \
  do {                                                                                  \
    const uint32_t la_ = Ls[ST] + (uint32_t)(TLPW * wave) * 1024u;                      \
    const uint32_t lb_ = Ls[ST] + TBM * CH * 16 + (uint32_t)(LPWB * wave) * 1024u;      \
    _Pragma("unroll") for (int j = 0; j < TLPW; ++j) {                                  \
      if (WIDE) lds_dma16(aptr[WIDE ? j : 0] + (K0) * 2, la_ + j * 1024);               \
      else lds_dma16(MOE_AADDR(K0), aoff[j], la_ + j * 1024);                           \
    }                                                                                   \
    _Pragma("unroll") for (int j = 0; j < LPWB; ++j)                                    \
      lds_dma16(MOE_BADDR(K0), boff[j], lb_ + j * 1024);                                \
  } while (0)
#define MOE_LOADF(SLOT, ST, KS, MIA) \
  do {                               \
    MOE_LOADA(SLOT, ST, KS, MIA);    \
    MOE_LOADB(SLOT, ST, KS);         \
  } while (0)
// operands of k-contiguous tiles ([row][MBK k], 16-byte chunk XOR swizzles)
#define MOE_LOADA_ROWS(SLOT, ST, KS, MIA)                                              \
  do {                                                                                 \
    const int chunk_ = (KS) * 2 + (lane >> 5);                                         \
    _Pragma("unroll") for (int mi = 0; mi < (MIA); ++mi) fa[SLOT][mi] = as_bf16x8(     \
        SA[ST][arow[mi] * CH + (chunk_ ^ ((arow[mi] >> 1) & 7))]);                     \
  } while (0)
#define MOE_LOADB_ROWS(SLOT, ST, KS)                                                   \
  do {                                                                                 \
    const int chunk_ = (KS) * 2 + (lane >> 5);                                         \
    if (I8) {                                                                          \
      _Pragma("unroll") for (int s = 0; s < NI; ++s) {                                 \
        const uint2 q_ = reinterpret_cast<const uint2*>(                               \
            SB[ST] + brow[s] * BCH + ((KS) ^ ((brow[s] >> 2) & 3)))[lane >> 5];        \
        fb[SLOT][s] = as_bf16x8(i8x8_to_bf16x8(q_.x, q_.y));                           \
      }                                                                                \
    } else {                                                                           \
      _Pragma("unroll") for (int s = 0; s < NI; ++s) fb[SLOT][s] = as_bf16x8(          \
          SB[ST][brow[s] * BCH + (chunk_ ^ ((brow[s] >> 1) & 7))]);                    \
    }                                                                                  \
  } while (0)
// operands of k-major tiles ([MBK k][256 columns], see kmajor_frag)
#define MOE_LOADA_KMAJOR(SLOT, ST, KS, MIA)                                            \
  do {                                                                                 \
    _Pragma("unroll") for (int mi = 0; mi < (MIA); ++mi) fa[SLOT][mi] =                \
        kmajor_frag(Ls[ST], acol[mi], (KS), lane);                                     \
  } while (0)
#define MOE_LOADB_KMAJOR(SLOT, ST, KS)                                                 \
  do {                                                                                 \
    _Pragma("unroll") for (int s = 0; s < NI; ++s) fb[SLOT][s] =                       \
        kmajor_frag(Ls[ST] + TBM * CH * 16, bcol[s], (KS), lane);                      \
  } while (0)
// Stage kt lives in buffer kt % NST. The first NST stages are issued up
// front; after stage kt is computed, once stage kt+1 has landed for every
// wave (later stages may still be in flight) and nobody reads stage kt any
// more, its buffer is refilled with stage kt + NST. A do-while keeps the
// compiler from carrying a zero-trip copy of the accumulators across the loop.
#define MOE_PIPELINE(KT_, MIA)                                                            \
  do {                                                                                    \
    const int KT = (KT_);                                                                 \
    _Pragma("unroll") for (int s_ = 0; s_ < NST; ++s_)                                    \
      if (s_ < KT) MOE_ISSUE(s_, s_ * MBK);                                                \
    wait_landed<TLPW + LPWB>(min(NST - 1, KT - 1));                                       \
    block_sync();                                                                         \
    MOE_LOADF(0, 0, 0, MIA);                                                              \
    int kt0 = 0;                                                                          \
    do {                                                                                  \
      _Pragma("unroll") for (int u = 0; u < NST; ++u) {                                   \
        const int kt = kt0 + u;                                                           \
        if (kt < KT) {                                                                    \
          _Pragma("unroll") for (int ks = 0; ks < NKS; ++ks) {                            \
            const int slot = ks & 1;                                                      \
            if (ks + 1 < NKS) {                                                           \
              MOE_LOADF(slot ^ 1, u, ks + 1, MIA);                                        \
            } else if (kt + 1 < KT) {                                                     \
              wait_landed<TLPW + LPWB>(min(NST - 2, KT - 2 - kt));                        \
              wait_lgkmcnt0();                                                            \
              block_sync();                                                               \
              if (kt + NST < KT) MOE_ISSUE(u, (kt + NST) * MBK);                          \
              MOE_LOADF(slot ^ 1, (u + 1) % NST, 0, MIA);                                 \
            }                                                                             \
            MOE_PRE_MFMA(slot, kt, ks);                                                   \
            _Pragma("unroll") for (int mi = 0; mi < (MIA); ++mi)                          \
              _Pragma("unroll") for (int s = 0; s < NI; ++s)                              \
                acc[mi][s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                     \
                    fa[slot][mi], fb[slot][s], acc[mi][s], 0, 0, 0);                      \
            /* one MFMA, then MOE_READS_AFTER(q, MIA) LDS reads of the next step */       \
            _Pragma("unroll") for (int q = 0; q < (MIA) * NI; ++q) {                      \
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          \
              _Pragma("unroll") for (int r_ = 0; r_ < MOE_READS_AFTER(q, MIA); ++r_)      \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                        \
            }                                                                             \
          }                                                                               \
        }                                                                                 \
      }                                                                                   \
      kt0 += NST;                                                                         \
    } while (kt0 < KT);                                                                   \
  } while (0)

// k-major tiles: MBK rows of k, each 256 bf16 columns (512 bytes, 32 chunks
// of 16 bytes); chunk c of row r sits at chunk c ^ kswz(r). An MFMA operand
// (lane l: 8 consecutive k of column colbase + l % 32, k = 16 ks + 8 (l / 32)
// + 0..7) comes from two ds_read_b64_tr_b16: in each group of 16 lanes, lane
// j points at 4 columns (colbase + 16 (g % 2) + 4 (j % 4), g = l / 16) of row
// 16 ks + 8 (g / 2) + j / 4 (+ 4 for the second read), and the read hands
// lane i of the group the 4 values of column i from those 4 rows. The 8 rows
// of one read then carry 8 distinct swizzles, so its 64-byte pieces land in
// 8 distinct 64-byte bank groups.
MOE_DEV int kswz(int r) { return ((r & 3) + 4 * ((r >> 3) & 1)) * 4; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

MOE_DEV bf16x8 kmajor_frag(uint32_t tile, int colbase, int ks, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int r = ks * 16 + 8 * (g >> 1) + (j >> 2);
  const int col = colbase + 16 * (g & 1) + 4 * (j & 3);
  // rows r and r + 4 share a swizzle (r % 4 and r / 8 agree)
  const uint32_t off = (uint32_t)(((col >> 3) ^ kswz(r)) * 16 + (col & 7) * 2);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<lds_s16x4*>((uintptr_t)(tile + (uint32_t)r * 512u + off)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<lds_s16x4*>((uintptr_t)(tile + (uint32_t)(r + 4) * 512u + off)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Zero the k positions of an operand at or past `valid` (stage-relative):
// lane l holds k = 16 ks + 8 (l / 32) + 0..7.
MOE_DEV bf16x8 mask_k(bf16x8 v, int ks, int lane, int valid) {
  const int n = valid - (ks * 16 + 8 * (lane >> 5));   // valid entries among the 8
  u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t keep = n >= 2 * q + 2 ? 0xffffffffu : n == 2 * q + 1 ? 0x0000ffffu : 0u;
    w[q] &= keep;
  }
  return __builtin_bit_cast(bf16x8, w);
}

// Output staging through LDS. Written straight from the 32x32 accumulator
// layout, a 256 x 256 bf16 tile takes 128 two-byte stores per wave, and the
// store instructions, not the bytes, bound the epilogue. Instead the tile
// goes to the two LDS stages column-major ([n][m]: 256 rows of 512 bytes,
// n < 128 in stage 0), each lane writing its 4 consecutive m of one column
// as one 8-byte slot; slot (m / 4) of row n sits at (m / 4) ^ stage_swz(n).
// Each lane then gathers 8 consecutive n of one m with two transposing
// reads and writes them with one 16-byte store (16 per wave). Writes: the
// 32 lanes of a half-wave cover 32 consecutive n at one m / 4, 32 distinct
// slots mod 32, so all 64 banks once. Reads: 16-lane group g of a read
// covers n = base + 32 g + 8 q + e (q, e < 4, +4 for the second read): the
// low 4 bits of stage_swz take n's bits 0, 1, 3, 4 and bit 4 takes bit 2 ^
// bit 5, so two groups again cover 32 distinct slots.
MOE_DEV int stage_swz(int n) {
  const int l = n & 31;
  return ((l & 3) | ((l >> 1) & 0xC) | ((l & 4) << 2)) ^ (((n >> 5) & 1) << 4);
}
MOE_DEV uint32_t stage_addr(uint32_t L0, uint32_t L1, int n, int mq) {
  return (n < 128 ? L0 + (uint32_t)n * 512u : L1 + (uint32_t)(n - 128) * 512u) +
         (uint32_t)((mq ^ stage_swz(n)) * 8);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
// rows 4 mq + 0..3 of column n (tile-local)
MOE_DEV void stage_put4(uint32_t L0, uint32_t L1, int n, int mq, float a, float b, float c,
                        float d) {
  const u32x2 v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  *reinterpret_cast<lds_u32x2*>((uintptr_t)stage_addr(L0, L1, n, mq)) = v;
}
// Read back for (mq, nb): this lane gets row 4 mq + (lane & 3), columns
// nb + 32 (lane / 16) + 8 ((lane / 4) & 3) + 0..7 (returned via col).
MOE_DEV uint4 stage_get8(uint32_t L0, uint32_t L1, int mq, int nb, int lane, int& row, int& col) {
  const int g = lane >> 4, i = lane & 15;
  // as a source of the transposing read: lane i points at n = ... + 8 (i % 4) + i / 4
  const int n = nb + 32 * g + 8 * (i & 3) + (i >> 2);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<lds_s16x4*>((uintptr_t)stage_addr(L0, L1, n, mq)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<lds_s16x4*>((uintptr_t)stage_addr(L0, L1, n + 4, mq)));
  row = 4 * mq + (i & 3);
  col = nb + 32 * g + 8 * (i >> 2);
  uint4 v;
  v.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  v.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  v.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  v.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return v;
}
// every wave's LDS operand reads and direct loads done, then a barrier
MOE_DEV void stage_begin() {
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  block_sync();
}
// the staged tile written, before the read-back
MOE_DEV void stage_mid() {
  wait_lgkmcnt0();
  block_sync();
}

// WIDE: the gathered activation rows are addressed with 64-bit per-lane
// pointers (x larger than 2 GiB); otherwise with 32-bit offsets from x.
// Tile shapes (TBM activation rows x BN weight rows): the wide tiles, 256 x
// 256, for experts with more than kStreamRows rows; the stream tiles, 128 x
// 512, for experts with at most kStreamRows rows (one row tile each), whose
// weights are read once per launch from HBM while their few activation rows
// are re-read from L2 for each column tile: the wider the tile, the fewer
// those re-reads (two stages of 16 + 64 KB fill the 160 KB of LDS).
// CLS: which experts the launch covers (kClsAll, kClsStream, kClsWide).
template <int MODE, int WT, bool WIDE, int TBM, int BN>
__global__ __launch_bounds__(MNW * 64) void ffn_mfma_kernel(FfnArgs a, uint32_t n_ntiles,
                                                            int cls) {
  constexpr bool GATEUP = MODE == M_GATEUP || MODE == M_GATEUP_SAVE;
  constexpr bool I8 = WT == WT_I8;
  constexpr int NST = 2;
  constexpr int TLPW = TBM * 8 / 64 / MNW;     // A LDS-DMA loads per wave per stage
  constexpr int ESZ = BTile<WT, BN>::ESZ, BCH = BTile<WT, BN>::BCH, LPWB = BTile<WT, BN>::LPW;
  constexpr int CH = MBK / 8;                   // 16-byte chunks per A row (bf16)
  constexpr int MWM = WaveGrid<WT, TBM, BN>::M, MWN = WaveGrid<WT, TBM, BN>::N;
  constexpr int NWR = BN / MWN;                 // weight rows per wave
  constexpr int MI = TBM / MWM / 32, NI = NWR / 32;
  constexpr int NKS = MBK / 16;
  static_assert(MI >= 2 && MI % 2 == 0, "a half tile takes half of each wave's row blocks");
  static_assert(!GATEUP || NI % 2 == 0, "a wave takes gate and up blocks in pairs");
  static_assert(TBM * BN <= MBM * MNB, "a split piece's partial tile fits one scratch slot");
  // one LDS variable per stage: the A tile then the B tile
  constexpr int STG = TBM * CH + BN * BCH;
  __shared__ u32x4 sT0[STG], sT1[STG];
  u32x4* const SA[2] = {sT0, sT1};
  u32x4* const SB[2] = {sT0 + TBM * CH, sT1 + TBM * CH};
  const uint32_t Ls[2] = {lds_addr(sT0), lds_addr(sT1)};

  const int N = GATEUP ? a.F : a.H;
  const int K = GATEUP ? a.H : a.F;
  uint32_t lin, pslot = 0;
  int piece = -1, npieces = 1;
  GroupedTile tile;
  if (GATEUP) {
    // (with 128 output columns per wide tile the Grok-1 shape's 256 column
    // tiles fill whole rounds of every XCD)
    if (!xcd_tile_index(a.offsets, a.E, TBM, n_ntiles, cls, lin)) return;
  } else {
    if (!xcd_tail_work(a.offsets, a.E, TBM, n_ntiles, cls, K / MBK, lin, piece, npieces, pslot))
      return;
  }
  if (!grouped_tile(a.offsets, a.E, TBM, n_ntiles, cls, lin, tile)) return;
  // k stages of this work item (a piece of a split tail tile, or all)
  const int kb = piece >= 0 ? piece * (K / MBK) / npieces : 0;
  const int ke = piece >= 0 ? (piece + 1) * (K / MBK) / npieces : K / MBK;
  constexpr int BNO = GATEUP ? BN / 2 : BN;  // output columns per tile
  const int e = __builtin_amdgcn_readfirstlane(tile.e);
  const int m0 = __builtin_amdgcn_readfirstlane(tile.m0);
  const int m_end = __builtin_amdgcn_readfirstlane(tile.m_end);
  const int n0 = __builtin_amdgcn_readfirstlane(tile.nt * BNO);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Swizzles. A (bf16, 8 chunks per row): chunk c of row r sits at physical
  // chunk c ^ ((r >> 1) & 7). B int8 (4 chunks per row): c ^ ((r >> 2) & 3).
  // Either way the 16 rows read by one 16-lane group hit 16 distinct banks.
  //
  // A: gathered x rows (gate/up) or this tile's h rows (down). The k offset
  // goes into the scalar base.
  const char* const abase = GATEUP ? uniform_ptr(a.x)
                                   : uniform_ptr(static_cast<const char*>(a.h) +
                                                 (int64_t)m0 * a.F * 2 + (int64_t)kb * MBK * 2);
  uint32_t aoff[TLPW];
  const char* aptr[WIDE ? TLPW : 1];
#pragma unroll
  for (int j = 0; j < TLPW; ++j) {
    const int q = (TLPW * wave + j) * 64 + lane;
    const int r = q / CH, c = (q % CH) ^ ((r >> 1) & 7);
    const int row = min(m0 + r, m_end - 1);
    if (GATEUP) {
      const int64_t tok = a.perm[row] / a.k;
      if (WIDE) aptr[WIDE ? j : 0] = static_cast<const char*>(a.x) + tok * a.H * 2 + c * 16;
      else aoff[j] = (uint32_t)tok * (uint32_t)(a.H * 2) + c * 16;
    } else {
      aoff[j] = (uint32_t)(row - m0) * (uint32_t)(a.F * 2) + c * 16;
    }
  }
  // B: one weight matrix per wave. Each wave loads consecutive B-tile rows;
  // with GATEUP, waves [0, MNW/2) load the gate rows (tile rows [0, BN/2))
  // and the others the up rows of the same output columns.
  const void* const wmat = GATEUP ? (wave < MNW / 2 ? a.wg : a.wu) : a.wd;
  const char* const bbase = uniform_ptr(static_cast<const char*>(wmat) +
                                        (((int64_t)e * N + n0) * K + (int64_t)kb * MBK) * ESZ);
  uint32_t boff[LPWB];
#pragma unroll
  for (int j = 0; j < LPWB; ++j) {
    const int q = (LPWB * wave + j) * 64 + lane;
    const int r = q / BCH;
    const int c = I8 ? (q % BCH) ^ ((r >> 2) & 3) : (q % BCH) ^ ((r >> 1) & 7);
    const int rr = GATEUP ? (r & (BN / 2 - 1)) : r;
    const int n = min(n0 + rr, N - 1) - n0;
    boff[j] = (uint32_t)n * (uint32_t)(K * ESZ) + c * 16;
  }

  // Rows: wave (wm, wn) owns the row blocks mi * RB + wm * 32 .. + 31 (RB =
  // 32 * MWM, mi < MI). The blocks of all waves interleave, so that in a
  // partial tile (an expert's last) the blocks that hold no row are spread
  // over the waves: a wave whose rows fit its first MI / 2 blocks skips the
  // MFMAs of the others. Waves w and w + 4 share a SIMD, so a wide bf16 tile
  // of at most 128 rows halves every SIMD's MFMA work, one of at most 192
  // rows cuts the busiest SIMD's by a quarter.
  constexpr int RB = 32 * MWM;
  const int wm = wave / MWN, wn = wave % MWN;
  int arow[MI], brow[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) arow[mi] = mi * RB + wm * 32 + (lane & 31);
#pragma unroll
  for (int s = 0; s < NI; ++s)
    brow[s] = (GATEUP ? (s < NI / 2 ? wn * (NWR / 2) + s * 32
                                    : BN / 2 + wn * (NWR / 2) + (s - NI / 2) * 32)
                      : wn * NWR + s * 32) + (lane & 31);
  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int s = 0; s < NI; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][s][v] = 0.f;
  bf16x8 fa[2][MI], fb[2][NI];

  // K >= 64 and a piece holds >= 1 stage, so there is at least one stage
#define MOE_AADDR(K0) (abase + (K0) * 2)
#define MOE_BADDR(K0) (bbase + (K0) * ESZ)
#define MOE_LOADA MOE_LOADA_ROWS
#define MOE_LOADB MOE_LOADB_ROWS
#define MOE_PRE_MFMA(SLOT, KT_, KS)
#define MOE_READS_AFTER(q, MIA) ((q) < (MIA) + NI ? 1 : 0)
  // row blocks of this wave that start before the tile's end (they come first)
  int mia = 0;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
    if (m0 + mi * RB + wm * 32 < m_end) mia = mi + 1;
  if (mia <= MI / 2) MOE_PIPELINE(ke - kb, MI / 2);
  else MOE_PIPELINE(ke - kb, MI);
#undef MOE_AADDR
#undef MOE_BADDR
#undef MOE_LOADA
#undef MOE_LOADB
#undef MOE_PRE_MFMA
#undef MOE_READS_AFTER

  // epilogue; 32x32 accumulator layout: lane l holds column l%32, register
  // v holds row 8*(v/4) + 4*(l/32) + v%4 of the block (rows past m_end,
  // including the blocks a half tile skipped, are not written)
  const int jcol = lane & 31;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = m0 + mi * RB + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (r >= m_end) continue;
      if (GATEUP) {
        uint16_t* hrow = static_cast<uint16_t*>(a.h) + (int64_t)r * a.F;
#pragma unroll
        for (int si = 0; si < NI / 2; ++si) {
          const int n = n0 + wn * (NWR / 2) + si * 32 + jcol;
          if (n < N) {
            float g = acc[mi][si][v], u = acc[mi][si + NI / 2][v];
            if (I8) {
              g *= a.sg[(int64_t)e * a.F + n];
              u *= a.su[(int64_t)e * a.F + n];
            }
            hrow[n] = f32_to_bf16_bits(swiglu(g, u));
            if (MODE == M_GATEUP_SAVE) {
              static_cast<uint16_t*>(a.g_save)[(int64_t)r * a.F + n] = f32_to_bf16_bits(g);
              static_cast<uint16_t*>(a.u_save)[(int64_t)r * a.F + n] = f32_to_bf16_bits(u);
            }
          }
        }
      } else if (piece >= 0) {
        // a piece of a split tail tile: float32 partial tile [TBM][BN],
        // summed (and scaled) by tail_reduce_kernel
        float* prow = static_cast<float*>(a.ws) + (int64_t)pslot * MBM * MNB + (r - m0) * BN;
#pragma unroll
        for (int s = 0; s < NI; ++s) prow[wn * NWR + s * 32 + jcol] = acc[mi][s][v];
      } else {
        uint16_t* yrow = static_cast<uint16_t*>(a.y) + (int64_t)r * a.H;
#pragma unroll
        for (int s = 0; s < NI; ++s) {
          const int n = n0 + wn * NWR + s * 32 + jcol;
          if (n < N)
            yrow[n] = f32_to_bf16_bits(I8 ? acc[mi][s][v] * a.sd[(int64_t)e * a.H + n]
                                          : acc[mi][s][v]);
        }
      }
    }
  }
}

// The split tail tiles of a tail-split launch (the down projection, the data
// gradients): y[r][n] = the pieces' float32 partials summed in piece order
// (times scale[e][n] when scale is set), rounded once to bf16. A tail tile
// (TBM x BN, in a scratch slot of MBM x MNB floats) is reduced by
// kReduceParts work-groups, one float4 of it per thread.
struct TailReduce {
  const int32_t* offsets;
  int E;
  int N;          // columns of y
  int kstages;    // k stages of a whole tile (bounds the pieces)
  const float* ws;
  void* y;        // [rows][N] bf16
  const float* scale;   // [E][N] or null
  int cls;        // the launch's expert class
};
constexpr int kReduceParts = MBM * MNB / 4 / 256;

template <int TBM, int BN>
__global__ __launch_bounds__(256) void tail_reduce_kernel(TailReduce t, uint32_t n_ntiles) {
  const uint32_t part = blockIdx.x % kReduceParts, tj = blockIdx.x / kReduceParts;
  const uint32_t xcd = tj / kCusPerXcd, j = tj % kCusPerXcd;
  const TailPlan p = tail_plan(t.offsets, t.E, TBM, n_ntiles, t.cls, xcd, t.kstages);
  if (p.S <= 1 || j >= p.tail) return;
  GroupedTile tile;
  if (!grouped_tile(t.offsets, t.E, TBM, n_ntiles, t.cls, p.base + p.full + j, tile)) return;
  const float4* src0 = reinterpret_cast<const float4*>(t.ws) +
                       (int64_t)(xcd * kTailSlots + j * p.S) * (MBM * MNB / 4);
  static_assert(TBM * BN == MBM * MNB, "one float4 of the tile per thread");
  {
    const int q = (int)part * 256 + (int)threadIdx.x;   // float4 of the tile
    const int r = tile.m0 + q / (BN / 4), n = tile.nt * BN + (q % (BN / 4)) * 4;
    if (r >= tile.m_end || n >= t.N) return;
    const float4* src = src0 + q;
    float4 v = src[0];
#pragma unroll
    for (uint32_t pc = 1; pc < kTailMaxPieces; ++pc) {
      if (pc < p.S) {
        const float4 w = src[(int64_t)pc * (MBM * MNB / 4)];
        v.x += w.x;
        v.y += w.y;
        v.z += w.z;
        v.w += w.w;
      }
    }
    const float o[4] = {v.x, v.y, v.z, v.w};
    uint16_t* yrow = static_cast<uint16_t*>(t.y) + (int64_t)r * t.N;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (n + c >= t.N) break;
      const float sc = t.scale ? t.scale[(int64_t)tile.e * t.N + n + c] : 1.f;
      yrow[n + c] = f32_to_bf16_bits(t.scale ? o[c] * sc : o[c]);
    }
  }
}

template <int TBM, int BN>
hipError_t launch_tail_reduce(const TailReduce& t, uint32_t n_ntiles, hipStream_t s) {
  hipLaunchKernelGGL((tail_reduce_kernel<TBM, BN>), dim3(8 * kCusPerXcd * kReduceParts),
                     dim3(256), 0, s, t, n_ntiles);
  return hipGetLastError();
}

// One launch of the forward GEMM over one class of experts (and, for the
// down projection, the reduce of its split tail tiles).
template <int MODE, int WT, bool WIDE, int TBM, int BN>
hipError_t launch_mfma(const FfnArgs& a, int cls, hipStream_t s) {
  constexpr bool GATEUP = MODE == M_GATEUP || MODE == M_GATEUP_SAVE;
  const uint32_t nt = GATEUP ? (uint32_t)((a.F + BN / 2 - 1) / (BN / 2))
                             : (uint32_t)((a.H + BN - 1) / BN);
  // worst case: every assignment (stream class: one row tile per expert)
  const unsigned tiles = cls == kClsStream ? (unsigned)((a.E * nt + 7) / 8 * 8)
                                           : grouped_grid(a.T * a.k, a.E, TBM, nt);
  const unsigned grid = tiles + (GATEUP ? 0 : kTailExtraBlocks);
  hipLaunchKernelGGL((ffn_mfma_kernel<MODE, WT, WIDE, TBM, BN>), dim3(grid), dim3(MNW * 64), 0,
                     s, a, nt, cls);
  if (GATEUP) return hipGetLastError();
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const TailReduce t{a.offsets, a.E, a.H, a.F / MBK, static_cast<const float*>(a.ws), a.y,
                     WT == WT_I8 ? a.sd : nullptr, cls};
  return launch_tail_reduce<TBM, BN>(t, nt, s);
}

// The forward GEMM over all experts: those with more than kStreamRows rows on
// the wide tiles, those with at most kStreamRows rows on the stream tiles. The
// split is made on the device from the dispatch offsets (each launch's
// work-groups find their class's tiles there). Above a mean of
// kStreamMeanRows rows per expert (known on the host: T k / E) every expert
// takes the wide tiles: an expert with at most kStreamRows rows is then an
// outlier, and the two stream launches, empty in the common case, cost 30 to
// 85 us per layer (measured at 2048 and 8192 tokens).
constexpr int64_t kStreamMeanRows = 256;

template <int MODE, int WT, bool WIDE>
hipError_t launch_mfma_all(const FfnArgs& a, hipStream_t s) {
  if (a.T * a.k > (int64_t)a.E * kStreamMeanRows)
    return launch_mfma<MODE, WT, WIDE, MBM, MNB>(a, kClsAll, s);
  hipError_t e = launch_mfma<MODE, WT, WIDE, MBM, MNB>(a, kClsWide, s);
  if (e != hipSuccess) return e;
  return launch_mfma<MODE, WT, WIDE, kStreamRows, 2 * MNB>(a, kClsStream, s);
}

// ---------------------------------------------------------------------------
// backward products on operands as they lie in HBM (no transposed copies)
// ---------------------------------------------------------------------------
// Weight gradients: per expert e,
//   C_e[m][n] = sum over the expert's dispatch rows r of a[r][m] * b[r][n],
// both operands row-major over the dispatch rows (dy and h for dW_down,
// [dg | du] and the gathered x rows for dW_gate|dW_up), so both are k-major
// tiles read through transposing LDS reads. The last stage of an expert
// reads up to 63 rows past its end (the buffers keep 64 rows of slack after
// the last dispatch row); those k positions are zeroed in both operands
// before the MFMAs. Tiles: MT x NT per expert; a group of tiles that share one operand block
// (the MT m tiles of one n tile when m_fast, else the NT n tiles of one m
// tile) stays on one XCD, and the XCDs take groups in turn, so a heavy
// expert is spread over all of them. Rows m < m_split go to out0
// [E][m_split][N], the rest to out1 [E][M - m_split][N], bf16.
__global__ __launch_bounds__(MNW * 64) void wgrad_tn_kernel(WgradTnArgs w) {
  constexpr bool WIDE = false;
  constexpr int NST = 2;
  constexpr int CH = MBK / 8, NKS = MBK / 16;
  constexpr int BCH = BTile<WT_BF16, MNB>::BCH, LPWB = BTile<WT_BF16, MNB>::LPW;
  constexpr int MWM = WaveGrid<WT_BF16, MBM, MNB>::M, MWN = WaveGrid<WT_BF16, MBM, MNB>::N;
  constexpr int TBM = MBM, TLPW = MLPW;
  constexpr int MW = MBM / MWM, NWR = MNB / MWN;
  constexpr int MI = MW / 32, NI = NWR / 32;
  __shared__ u32x4 sT0[MBM * CH + MNB * BCH], sT1[MBM * CH + MNB * BCH];
  const uint32_t L0 = lds_addr(sT0), L1 = lds_addr(sT1);
  const uint32_t Ls[2] = {L0, L1};
  const char* const* aptr = nullptr;

  const uint32_t MT = (uint32_t)(w.M + MBM - 1) / MBM, NT = (uint32_t)(w.N + MNB - 1) / MNB;
  const uint32_t G = w.m_fast ? MT : NT;
  const uint32_t slot_ = blockIdx.x >> 3;
  const uint32_t lin = ((slot_ / G) * 8 + (blockIdx.x & 7)) * G + slot_ % G;
  if (lin >= (uint32_t)w.E * MT * NT) return;
  const int e = (int)(lin / (MT * NT));
  const uint32_t rem = lin % (MT * NT);
  const int mt = (int)(w.m_fast ? rem % MT : rem / NT);
  const int nt = (int)(w.m_fast ? rem / MT : rem % NT);
  const int m0 = mt * MBM, n0 = nt * MNB;
  const int r0 = __builtin_amdgcn_readfirstlane(w.offsets[e]);
  const int ne = __builtin_amdgcn_readfirstlane(w.offsets[e + 1]) - r0;
  const int kt = (ne + MBK - 1) / MBK;
  const int klast = ne - (kt - 1) * MBK;     // valid rows in the last stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const char* const abase = uniform_ptr(static_cast<const char*>(w.a) + (int64_t)r0 * w.lda * 2);
  const char* const bbase = uniform_ptr(static_cast<const char*>(w.b) + (int64_t)r0 * w.ldb * 2);
  uint32_t aoff[MLPW], boff[LPWB];
#pragma unroll
  for (int j = 0; j < MLPW; ++j) {
    const int q = (MLPW * wave + j) * 64 + lane;
    const int kk = q >> 5, c = (q & 31) ^ kswz(kk);
    aoff[j] = (uint32_t)kk * (uint32_t)(w.lda * 2) + (uint32_t)min(m0 + 8 * c, w.M - 8) * 2u;
  }
#pragma unroll
  for (int j = 0; j < LPWB; ++j) {
    const int q = (LPWB * wave + j) * 64 + lane;
    const int kk = q >> 5, c = (q & 31) ^ kswz(kk);
    boff[j] = (uint32_t)kk * (uint32_t)(w.ldb * 2) + (uint32_t)min(n0 + 8 * c, w.N - 8) * 2u;
  }
  const int wm = wave / MWN, wn = wave % MWN;
  int acol[MI], bcol[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) acol[mi] = wm * MW + mi * 32;
#pragma unroll
  for (int s = 0; s < NI; ++s) bcol[s] = wn * NWR + s * 32;
  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int s = 0; s < NI; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][s][v] = 0.f;
  bf16x8 fa[2][MI], fb[2][NI];

#define MOE_AADDR(K0) (abase + (int64_t)(K0) * w.lda * 2)
#define MOE_BADDR(K0) (bbase + (int64_t)(K0) * w.ldb * 2)
#define MOE_LOADA MOE_LOADA_KMAJOR
#define MOE_LOADB MOE_LOADB_KMAJOR
#define MOE_PRE_MFMA(SLOT, KT_, KS)                                              \
  do {                                                                           \
    if ((KT_) == KT - 1 && klast < MBK) {                                        \
      _Pragma("unroll") for (int mi = 0; mi < MI; ++mi)                          \
        fa[SLOT][mi] = mask_k(fa[SLOT][mi], (KS), lane, klast);                  \
      _Pragma("unroll") for (int s = 0; s < NI; ++s)                             \
        fb[SLOT][s] = mask_k(fb[SLOT][s], (KS), lane, klast);                    \
    }                                                                            \
  } while (0)
// 12 reads per step after 8 MFMAs (other placements measured the same)
#define MOE_READS_AFTER(q, MIA) ((q) < 4 ? 2 : 1)
  // an expert without rows has a zero gradient: no stage, zeros written
  if (kt > 0) MOE_PIPELINE(kt, MI);
#undef MOE_AADDR
#undef MOE_BADDR
#undef MOE_LOADA
#undef MOE_LOADB
#undef MOE_PRE_MFMA
#undef MOE_READS_AFTER

  // epilogue through LDS (stage_put4 / stage_get8)
  stage_begin();
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int s = 0; s < NI; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        stage_put4(L0, L1, wn * NWR + s * 32 + (lane & 31), (wm * MW + mi * 32 + 8 * j) / 4 + (lane >> 5),
                   acc[mi][s][4 * j], acc[mi][s][4 * j + 1], acc[mi][s][4 * j + 2],
                   acc[mi][s][4 * j + 3]);
  stage_mid();
#pragma unroll 4
  for (int it = 0; it < MBM * MNB / (MNW * 64 * 8); ++it) {
    const int combo = it * MNW + wave;
    int r, c;
    const uint4 v = stage_get8(L0, L1, combo % (MBM / 4), combo / (MBM / 4) * 128, lane, r, c);
    const int m = m0 + r, n = n0 + c;
    if (m >= w.M || n >= w.N) continue;
    uint16_t* const crow =
        m < w.m_split
            ? static_cast<uint16_t*>(w.out0) + ((int64_t)e * w.m_split + m) * w.N
            : static_cast<uint16_t*>(w.out1) +
                  ((int64_t)e * (w.M - w.m_split) + (m - w.m_split)) * w.N;
    *reinterpret_cast<uint4*>(crow + n) = v;
  }
}

// Data gradients: y[r][n] = sum_k a[r][k] * W_e[k][n] over the dispatch rows
// r of each expert, with the weight used as it is stored (k-major rows:
// W_down[e] is [H][F] for dh = dy W_down; for the dx rows, k < ksplit reads
// W_gate[e] [F][H] and k >= ksplit W_up[e], against a = [dg | du]). The A
// operand and the tiles are the down-mode kernel's, tail split included; B is
// a k-major tile read through transposing LDS reads.
__global__ __launch_bounds__(MNW * 64) void dgrad_nn_kernel(DgradArgs d, uint32_t n_ntiles) {
  constexpr bool WIDE = false;
  constexpr int NST = 2;
  constexpr int CH = MBK / 8, NKS = MBK / 16;
  constexpr int BCH = BTile<WT_BF16, MNB>::BCH, LPWB = BTile<WT_BF16, MNB>::LPW;
  constexpr int MWM = WaveGrid<WT_BF16, MBM, MNB>::M, MWN = WaveGrid<WT_BF16, MBM, MNB>::N;
  constexpr int TBM = MBM, TLPW = MLPW;
  constexpr int MW = MBM / MWM, NWR = MNB / MWN;
  constexpr int MI = MW / 32, NI = NWR / 32;
  __shared__ u32x4 sT0[MBM * CH + MNB * BCH], sT1[MBM * CH + MNB * BCH];
  u32x4* const SA[2] = {sT0, sT1};
  const uint32_t Ls[2] = {lds_addr(sT0), lds_addr(sT1)};
  const char* const* aptr = nullptr;

  uint32_t lin, pslot = 0;
  int piece = -1, npieces = 1;
  GroupedTile tile;
  if (!xcd_tail_work(d.offsets, d.E, MBM, n_ntiles, kClsAll, d.K / MBK, lin, piece, npieces,
                     pslot))
    return;
  if (!grouped_tile(d.offsets, d.E, MBM, n_ntiles, kClsAll, lin, tile)) return;
  // k range of this work item (a piece of a split tail tile, or all)
  const int kb = piece >= 0 ? piece * (d.K / MBK) / npieces : 0;
  const int ke = piece >= 0 ? (piece + 1) * (d.K / MBK) / npieces : d.K / MBK;
  const int kofs = kb * MBK;
  const int e = __builtin_amdgcn_readfirstlane(tile.e);
  const int m0 = __builtin_amdgcn_readfirstlane(tile.m0);
  const int m_end = __builtin_amdgcn_readfirstlane(tile.m_end);
  const int n0 = __builtin_amdgcn_readfirstlane(tile.nt * MNB);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const char* const abase =
      uniform_ptr(static_cast<const char*>(d.a) + (int64_t)m0 * d.K * 2 + (int64_t)kofs * 2);
  uint32_t aoff[MLPW];
#pragma unroll
  for (int j = 0; j < MLPW; ++j) {
    const int q = (MLPW * wave + j) * 64 + lane;
    const int r = q / CH, c = (q % CH) ^ ((r >> 1) & 7);
    aoff[j] = (uint32_t)(min(m0 + r, m_end - 1) - m0) * (uint32_t)(d.K * 2) + c * 16;
  }
  const char* const b0 = uniform_ptr(static_cast<const char*>(d.b0) +
                                     (int64_t)e * d.ksplit * d.N * 2);
  const char* const b1 = uniform_ptr(static_cast<const char*>(d.b1 ? d.b1 : d.b0) +
                                     (int64_t)e * (d.K - d.ksplit) * d.N * 2);
  uint32_t boff[LPWB];
#pragma unroll
  for (int j = 0; j < LPWB; ++j) {
    const int q = (LPWB * wave + j) * 64 + lane;
    const int kk = q >> 5, c = (q & 31) ^ kswz(kk);
    boff[j] = (uint32_t)kk * (uint32_t)(d.N * 2) + (uint32_t)min(n0 + 8 * c, d.N - 8) * 2u;
  }
  const int wm = wave / MWN, wn = wave % MWN;
  int arow[MI], bcol[NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) arow[mi] = wm * MW + mi * 32 + (lane & 31);
#pragma unroll
  for (int s = 0; s < NI; ++s) bcol[s] = wn * NWR + s * 32;
  f32x16 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int s = 0; s < NI; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][s][v] = 0.f;
  bf16x8 fa[2][MI], fb[2][NI];

#define MOE_AADDR(K0) (abase + (K0) * 2)
#define MOE_BADDR(K0)                                                          \
  ((K0) + kofs < d.ksplit ? b0 + (int64_t)((K0) + kofs) * d.N * 2              \
                          : b1 + (int64_t)((K0) + kofs - d.ksplit) * d.N * 2)
#define MOE_LOADA MOE_LOADA_ROWS
#define MOE_LOADB MOE_LOADB_KMAJOR
#define MOE_PRE_MFMA(SLOT, KT_, KS)
#define MOE_READS_AFTER(q, MIA) ((q) + MI * NI < MI + 2 * NI ? 2 : (q) < MI + 2 * NI ? 1 : 0)
  MOE_PIPELINE(ke - kb, MI);
#undef MOE_AADDR
#undef MOE_BADDR
#undef MOE_LOADA
#undef MOE_LOADB
#undef MOE_PRE_MFMA
#undef MOE_READS_AFTER

  const int jcol = lane & 31;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = m0 + wm * MW + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (r >= m_end) continue;
      if (piece >= 0) {
        float* prow = static_cast<float*>(d.ws) + (int64_t)pslot * MBM * MNB + (r - m0) * MNB;
#pragma unroll
        for (int s = 0; s < NI; ++s) prow[wn * NWR + s * 32 + jcol] = acc[mi][s][v];
        continue;
      }
      uint16_t* yrow = static_cast<uint16_t*>(d.y) + (int64_t)r * d.N;
#pragma unroll
      for (int s = 0; s < NI; ++s) {
        const int n = n0 + wn * NWR + s * 32 + jcol;
        if (n < d.N) yrow[n] = f32_to_bf16_bits(acc[mi][s][v]);
      }
    }
  }
}

#undef MOE_PIPELINE
#undef MOE_ISSUE
#undef MOE_LOADF
#undef MOE_LOADA_ROWS
#undef MOE_LOADB_ROWS
#undef MOE_LOADA_KMAJOR
#undef MOE_LOADB_KMAJOR

// 32-bit offsets from x reach the gathered rows while x is below 2 GiB
bool x_needs_wide(const FfnArgs& a) { return (uint64_t)a.T * (uint64_t)a.H * 2 > (1ull << 31); }

}  // namespace

size_t ffn_ws_bytes(int64_t T, int H, int F, int E, int k, Act act, Wt wt) {
  (void)F; (void)E; (void)wt;
  // float32 split-k partials of the down projection: every tile's on the
  // decode path, the split tail tiles' on the tiled path
  if (act != ACT_BF16) return 0;
  return T <= kDecodeMaxT ? decode_ws_bytes(T, H, k) : tiled_ws_bytes();
}

size_t tiled_ws_bytes() { return kTailScratchBytes; }

hipError_t launch_gateup_tiled(const FfnArgs& a, Wt wt, hipStream_t s) {
  if (wt == WT_I4) return hipErrorNotSupported;   // int4: decode kernels only
  if (x_needs_wide(a))
    return wt == WT_I8 ? launch_mfma_all<M_GATEUP, WT_I8, true>(a, s)
                       : launch_mfma_all<M_GATEUP, WT_BF16, true>(a, s);
  return wt == WT_I8 ? launch_mfma_all<M_GATEUP, WT_I8, false>(a, s)
                     : launch_mfma_all<M_GATEUP, WT_BF16, false>(a, s);
}

hipError_t launch_down_tiled(const FfnArgs& a, Wt wt, hipStream_t s) {
  if (wt == WT_I4) return hipErrorNotSupported;
  return wt == WT_I8 ? launch_mfma_all<M_DOWN, WT_I8, false>(a, s)
                     : launch_mfma_all<M_DOWN, WT_BF16, false>(a, s);
}

hipError_t launch_gateup_save_tiled(const FfnArgs& a, hipStream_t s) {
  return x_needs_wide(a) ? launch_mfma_all<M_GATEUP_SAVE, WT_BF16, true>(a, s)
                         : launch_mfma_all<M_GATEUP_SAVE, WT_BF16, false>(a, s);
}

hipError_t launch_wgrad_tn(const WgradTnArgs& w, hipStream_t s) {
  const unsigned MT = (unsigned)(w.M + MBM - 1) / MBM, NT = (unsigned)(w.N + MNB - 1) / MNB;
  const unsigned G = w.m_fast ? MT : NT;
  const unsigned groups = (unsigned)w.E * MT * NT / G;
  hipLaunchKernelGGL(wgrad_tn_kernel, dim3((groups + 7) / 8 * 8 * G), dim3(MNW * 64), 0, s, w);
  return hipGetLastError();
}

hipError_t launch_dgrad_nn(const DgradArgs& d, hipStream_t s) {
  const uint32_t nt = (uint32_t)((d.N + MNB - 1) / MNB);
  hipLaunchKernelGGL(dgrad_nn_kernel,
                     dim3(grouped_grid(d.T * d.k, d.E, MBM, nt) + kTailExtraBlocks),
                     dim3(MNW * 64), 0, s, d, nt);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const TailReduce t{d.offsets, d.E, d.N, d.K / MBK, static_cast<const float*>(d.ws), d.y,
                     nullptr, kClsAll};
  return launch_tail_reduce<MBM, MNB>(t, nt, s);
}


}  // namespace moe
