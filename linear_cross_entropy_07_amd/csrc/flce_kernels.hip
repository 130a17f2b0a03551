// HIP kernels (gfx950 / CDNA4) for fused linear + cross-entropy, forward and backward.
//
// The computation follows the PR description of "[AOTAutograd] tweak min-cut partitioner to avoid
// saving softmax output" (PyTorch PR #126348): the linear layer gives the softmax input, per-row
// max and sum statistics are formed from it, only the label's entry is needed for the loss, and
// the backward pass rebuilds the softmax from the softmax input and the small max/sum tensors
// instead of reading a saved softmax output. Here that happens per BT chunk:
//
//   k_rowref  per row: a reference c = the (softcapped) label logit, one dot product of hidden and
//             the label's row of W, known before the logits exist.
//   k_fwd     Z^T tile = W_tile . X_tile^T on MFMA (bf16 -> fp32), epilogue: optional softcap, and per
//             (row, 128-wide V segment) a reference r = max(c, segment max - kRefSpan), the sum of
//             exp(s - r), and one 16-bit store per logit of q = exp(s - r) * (softcap derivative): the
//             softmax numerator against the row's reference (r = c but for segments more than
//             kRefSpan above it). q is stored in blocks of 256 rows x one K step of grad_hidden, so
//             that each K step of the backward GEMMs reads long contiguous runs. No [BT, V] tensor
//             exists.
//   k_lse     per row: lse from the segment statistics and the loss term; a row with a segment whose
//             reference lies above c gets the largest segment reference as its reference, its stored q
//             rescaled segment by segment to match (the usual rows do nothing more).
//   k_rowfix  per row: f = g exp(c - lse), so that dZ_v = f q_v for v != label; the label entry of
//             q becomes (p_y - 1) / f, computed from the exact label logit; and hidden_f = f hidden.
//   k_dx      grad_hidden chunk = f . (q . W) on MFMA (W read MN-contiguous, transposed by the LDS
//             transpose reads on its way to the matrix cores; f applied to each output row).
//   k_dw      grad_W (+)= q^T . hidden_f on MFMA; both operands read MN-contiguous and transposed the
//             same way; fp32 accumulation in place across chunks. A last wave of tiles under half
//             full is split along K into fp32 partials, which k_dw_tail adds in a fixed order.
// So the softmax is rebuilt from the stored softmax input and the small per-row max/sum statistics,
// and dlogits are never written: the backward GEMMs take q as it was stored and the per-row factor
// f enters by linearity (an output-row scale for grad_hidden, a scaled copy of the chunk's hidden
// rows for grad_W).
//
// One GEMM core serves the three products: 512 threads (8 waves of 64) compute a 256 x 256 tile,
// each wave a 128 x 64 part as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (or 32x32x2f32 for fp32
// inputs; FLCE_MFMA=16 selects 8 x 4 blocks of 16x16x32 instead). Operands reach LDS by DMA (buffer
// loads that write LDS directly) into a ring of kStages stages of kStepBytes of K per row,
// XOR-swizzled against bank conflicts, and the main loop's instruction order is fixed in the source:
// each MFMA is followed by the fragment reads and DMA loads assigned to it.
#include <mutex>

#include "flce_internal.h"

namespace flce {
namespace {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// GEMM block: a 256 x 256 output tile split over NW waves as 2 (M) x NW/2 (N). With 8 waves each
// wave owns 128 x 64 (128 accumulator registers) and two waves share each SIMD, which doubles the
// LDS request rate a SIMD sustains; with 4 waves each owns 128 x 128 (256 accumulators).
#ifndef FLCE_WAVES
#define FLCE_WAVES 8
#endif
constexpr int NW = FLCE_WAVES;
constexpr int NTHR = 64 * NW;    // threads per GEMM block
constexpr int TILE = kTile;      // 256
constexpr int WM = TILE / 2;     // wave tile rows (M): 128, one 128-wide V segment in the logits GEMM
constexpr int WN = TILE / (NW / 2);  // wave tile columns (N): 64 or 128
// MFMA block: 32 x 32 (v_mfma_f32_32x32x16_bf16, K = 16 per instruction) or 16 x 16
// (v_mfma_f32_16x16x32_bf16, K = 32). Both do the same flops per cycle on paper and read the same
// LDS bytes per flop here. On random data an MFMA-only loop of the 16 x 16 form sustains about 12%
// more under the chip's power limit (2.03 against 1.80 PF/s), but the three GEMMs measured even
// with it (within 1% per product), so the 32 x 32 form, with half the MFMA instructions, stays.
#ifndef FLCE_MFMA
#define FLCE_MFMA 32
#endif
constexpr int MB = FLCE_MFMA;    // edge of one MFMA output block
// DMA placement in the unrolled main loop: 0 issues a step's loads at its start; 1 (the default)
// spreads them, the first operand's loads one after each of a few MFMAs of the step's first substep
// and the second operand's one after each of a few MFMAs following the step's barrier. In the
// explicit order load d follows MFMA FLCE_DMA_FIRST + d * FLCE_DMA_STRIDE of its substep (MFMAs 2 and 4
// measured best on MI355X: after the substep's first fragment reads, before its last MFMAs).
#ifndef FLCE_DMA_SPREAD
#define FLCE_DMA_SPREAD 1
#endif
#ifndef FLCE_DMA_FIRST
#define FLCE_DMA_FIRST 2
#endif
#ifndef FLCE_DMA_STRIDE
#define FLCE_DMA_STRIDE 2
#endif
static_assert(MB == 16 || MB == 32, "16x16 or 32x32 MFMA blocks");
constexpr int NR = MB * MB / 64;  // accumulator registers per block and lane (4 or 16)
constexpr int TBM = WM / MB;     // MFMA blocks per wave tile along M (8 or 4)
constexpr int TBN = WN / MB;     // ... along N (4 or 2 with 8 waves)
static_assert(NW == 4 || NW == 8, "4 or 8 waves per GEMM block");
typedef float facc __attribute__((ext_vector_type(NR)));
// Accumulator layout: lane l holds column l % MB of its block and, in register r, row acc_row(r, l):
// 32 x 32: 8 (r / 4) + 4 (l / 32) + r % 4; 16 x 16: 4 (l / 16) + r. In both, registers 4g .. 4g+3
// are four consecutive rows, and acc_row(r, l) - acc_row(0, l) = acc_row(r, 0).
__device__ __forceinline__ int acc_row(int r, int lane) {
  return MB == 32 ? 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) : 4 * (lane >> 4) + r;
}
// 16-byte K chunk of a fragment read by this lane: 32 x 32 blocks take K 16 s .. 16 s + 15 per
// substep s, each lane half 8 of them; 16 x 16 blocks take K 0 .. 31 of the step, each 16-lane group
// 8 of them (one substep per step over K, split in two over the M blocks).
__device__ __forceinline__ int frag_chunk(int s, int lane) { return MB == 32 ? 2 * s + (lane >> 5) : (lane >> 4); }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
// q = exp(s - c) is stored against a per-row reference c; a segment whose maximum lies more than
// kRefSpan above c (only possible where the label logit lies that far below it) is stored against its
// maximum less kRefSpan instead, and its row is rescaled to one reference afterwards. Every stored q is
// thus at most exp(kRefSpan) = 7e20, which keeps q, and the fp32 sums of q times W over up to 2^20
// vocabulary rows, far from overflow.
constexpr float kRefSpan = 48.0f;

template <typename T> struct Traits;
template <> struct Traits<__bf16> {
  using S = __bf16;                   // workspace element type (q is an operand of the bf16 GEMMs)
  static constexpr int KV = 8;        // elements per 16-byte chunk
};
template <> struct Traits<float> {
  using S = float;
  static constexpr int KV = 4;
};

// Layout of q in the workspace: blocks of 256 chunk rows x kQB values (kStepBytes per row, one K
// step of the grad_hidden product), ordered by 256-row tile, then by v. A grad_hidden K step of one
// tile is then one contiguous 16 KiB block, and a grad_W K step (the tile's 256 v of a few chunk rows)
// is 256 / kQB runs of those rows. nkv = V_pad / kQB blocks per tile of rows.
template <typename S>
constexpr int kQB = kStepBytes / (int)sizeof(S);
template <typename S>
__host__ __device__ __forceinline__ int64_t q_index(int64_t c, int64_t v, int64_t nkv) {
  return (((c >> 8) * nkv + v / kQB<S>) * 256 + (c & 255)) * kQB<S> + v % kQB<S>;
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh from its definition through e^{2x}; saturates to +-1 for large |x|.
__device__ __forceinline__ float tanh_via_exp(float x) {
  const float e = ex2(2.0f * kLog2e * x);
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---- MFMA on one 16-byte chunk of K per lane --------------------------------------------------
#if FLCE_MFMA == 32
__device__ __forceinline__ void mma(facc& acc, u32x4 a, u32x4 b, __bf16*) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
#else
__device__ __forceinline__ void mma(facc& acc, u32x4 a, u32x4 b, __bf16*) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
#endif
__device__ __forceinline__ void mma(facc& acc, u32x4 a, u32x4 b, float*) {
  const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
  // each lane group (halves for 32 x 32, quarters for 16 x 16) holds 4 consecutive k of this K slice
  // in both operands; each of the four MFMAs pairs the e-th element of every group, so A and B see
  // the same k assignment.
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#if FLCE_MFMA == 32
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[e], fb[e], acc, 0, 0, 0);
#else
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[e], fb[e], acc, 0, 0, 0);
#endif
  }
}

// ---- 16-byte chunk conversions -------------------------------------------------------------
__device__ __forceinline__ void unpack(u32x4 v, float (&f)[8], __bf16*) {
  const f32x8 h = __builtin_convertvector(__builtin_bit_cast(bf16x8, v), f32x8);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = h[i];
}
__device__ __forceinline__ void unpack(u32x4 v, float (&f)[4], float*) {
  const f32x4 h = __builtin_bit_cast(f32x4, v);
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = h[i];
}
__device__ __forceinline__ u32x4 pack(const float (&f)[8], __bf16*) {
  f32x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = f[i];
  return __builtin_bit_cast(u32x4, __builtin_convertvector(v, bf16x8));  // round to nearest even
}
__device__ __forceinline__ u32x4 pack(const float (&f)[4], float*) {
  f32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = f[i];
  return __builtin_bit_cast(u32x4, v);
}
__device__ __forceinline__ u32x2 pack4_bf16(float a, float b, float c, float d) {
  return __builtin_bit_cast(u32x2, __builtin_convertvector((f32x4{a, b, c, d}), bf16x4));  // nearest even
}

// ---- block -> tile mapping -------------------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (block b on XCD b % 8). Give each XCD a
// contiguous run of the tile order so that tiles which share operand panels share one L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int xcd = b & 7, slot = b >> 3, q = nblocks >> 3, r = nblocks & 7;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}
// Grouped order: `gm` tile rows are swept together along N.
__device__ __forceinline__ void grouped(int t, int mt, int nt, int gm, int& tm, int& tn) {
  const int per = gm * nt, group = t / per, first = group * gm;
  const int gsz = min(mt - first, gm), in = t - group * per;
  tm = first + in % gsz;
  tn = in / gsz;
}

// ---- LDS DMA: global -> LDS without registers ------------------------------------------------
// buffer_load_dwordx4 ... lds writes each lane's 16 bytes to LDS at M0 + 16 * lane, so one wave
// instruction fills 1 KiB of LDS contiguously; the global address of each lane is free. The loads are
// issued from inline asm and their completion is awaited with explicit vmcnt waits, so that several
// stages can be in flight (the compiler's own tracking would wait for all of them before any LDS
// read). The buffer range makes out-of-range lanes write zeros, which covers every tile edge.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
constexpr u32 kOOB = 0x80000000u;  // an offset no buffer range here reaches (all ranges < 2 GiB)

__device__ __forceinline__ i32x4 make_desc(const void* base, u32 bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4{(int)__builtin_amdgcn_readfirstlane((u32)a), (int)__builtin_amdgcn_readfirstlane((u32)(a >> 32)),
               (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}
__device__ __forceinline__ u32 lds_addr(const void* p) {
  return (u32)(size_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ void dma16(i32x4 desc, u32 voff, u32 lds) {
  // M0 must be written one instruction before an LDS-DMA load reads it. M0 is a reserved register for
  // the compiler (never allocated; its own users write it right before they read it), so it cannot
  // appear in a clobber list and nothing the compiler emits relies on M0 across this statement.
#if FLCE_DMA_SPREAD
  // No memory clobber: fragment reads may be scheduled across the load. Every LDS byte a load writes
  // is read only after a later s_waitcnt + s_barrier statement, which does clobber memory, and the
  // slot it writes was last read before an earlier one; volatile statements keep their order.
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(desc), "s"(__builtin_amdgcn_readfirstlane(lds)));
#else
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(desc), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
#endif
}

// Range-checked buffer accesses for epilogues: loads outside the range return 0, stores outside it
// are dropped, so tile edges need no branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const u32 n = bytes <= 0 ? 0u : (u32)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(n), 0x00020000);
}
__device__ __forceinline__ void bstore_b64(rsrc_t r, u32 off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore_b128(rsrc_t r, u32 off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

// Accumulator addressing for row-major [rows][ld] output tiles whose element (0, 0) is the buffer
// base: a per-lane offset for each MB-column block j (kOOB past ncols) plus a wave-uniform row offset
// for (i, r), passed as the scalar offset of the buffer instruction. All tiles here keep
// row * ld * ESZ below 2^31, so 32-bit arithmetic is exact.
template <int ESZ>
struct AccAddr {
  u32 col[TBN];
  int ld;
  __device__ __forceinline__ AccAddr(int ld_, int ncols) : ld(ld_) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
    const int row0 = wm * WM + acc_row(0, lane);
#pragma unroll
    for (int j = 0; j < TBN; ++j) {
      const int c = wn * WN + MB * j + lane % MB;
      col[j] = c < ncols ? (u32)(row0 * ld + c) * (u32)ESZ : kOOB;
    }
  }
  __device__ __forceinline__ u32 row(int i, int r) const {
    return (u32)((MB * i + acc_row(r, 0)) * ld) * (u32)ESZ;
  }
};
__device__ __forceinline__ float bload_f32(rsrc_t r, u32 voff, u32 soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ void bstore_f32(rsrc_t r, u32 voff, u32 soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, v), r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void bstore_b16(rsrc_t r, u32 voff, u32 soff, unsigned short v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)voff, (int)soff, 0);
}

// ---- pipeline geometry ---------------------------------------------------------------------
// A stage holds kStepBytes of K for the 256 rows (or columns) of each operand.
constexpr int kChunks = kStepBytes / 16;           // 16-byte K chunks per row per step
constexpr int kSub = kChunks / 2;                  // MFMA substeps per step
constexpr int kStages = kPipeStages;
constexpr int kOpBytes = TILE * kStepBytes;        // per operand per stage
constexpr int kStageBytes = 2 * kOpBytes;          // A + B
constexpr int kDmaPerOp = kOpBytes / (NTHR * 16);  // DMA instructions per thread per operand
constexpr int kLoadsPerStage = 2 * kDmaPerOp;
constexpr bool kSpread = FLCE_DMA_SPREAD != 0;
static_assert(!kSpread || (kStages >= 3 && FLCE_DMA_FIRST + (kDmaPerOp - 1) * FLCE_DMA_STRIDE < TBM * TBN),
              "DMA spread: 3+ stages, every load after an MFMA of its substep");
static_assert(kChunks == 4 || kChunks == 8, "64 or 128 bytes of K per step");
static_assert(kStages >= 2 && kStages * kStageBytes <= 160 * 1024, "LDS ring must fit in 160 KiB");
// vmcnt field encoding of s_waitcnt (gfx9): low 4 bits and bits 15:14; expcnt and lgkmcnt left at max.
constexpr int vmcnt_only(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

// K-contiguous operand: tile row r (an M or N index) is a source row, K runs along it. In LDS each
// row holds kStepBytes (kChunks chunks of 16 bytes); chunk kc is stored at slot kc ^ swz(r), where
// swz changes every 256 bytes of rows, so that 16 rows read at one chunk index cover all banks.
// A fragment is one ds_read_b128.
template <typename T>
struct OpK {
  static constexpr int KV = 16 / sizeof(T), BK = kChunks * KV;
  static constexpr int RPI = 1024 / kStepBytes;  // rows per DMA instruction
  static __device__ __forceinline__ int swz(int row) { return (row / (256 / kStepBytes)) & (kChunks - 1); }
  i32x4 desc;          // rows [0, valid rows) of the tile
  u32 rowoff[kDmaPerOp];
  int kc[kDmaPerOp];   // chunk of K this lane loads for each of its rows
  int kmax;            // valid K elements (also the end of this block's K range)
  __device__ __forceinline__ void init(const T* p, int64_t ld, int rows, int kmax_) {
    desc = make_desc(p, (u32)(rows > 0 ? rows : 0) * (u32)(ld * sizeof(T)));
    kmax = kmax_;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kDmaPerOp; ++q) {
      const int row = RPI * (kDmaPerOp * wave + q) + lane / kChunks;
      rowoff[q] = (u32)(row * ld * (int64_t)sizeof(T));
      kc[q] = (lane % kChunks) ^ swz(row);
    }
  }
  __device__ __forceinline__ void issue_one(int ks, u32 lds, int q) const {
    const int wave = threadIdx.x >> 6;
    const int k = ks * BK + kc[q] * KV;
    dma16(desc, k < kmax ? rowoff[q] + (u32)(k * sizeof(T)) : kOOB, lds + (kDmaPerOp * wave + q) * 1024);
  }
  __device__ __forceinline__ void issue(int ks, u32 lds) const {
#pragma unroll
    for (int q = 0; q < kDmaPerOp; ++q) issue_one(ks, lds, q);
  }
  // fragment of rows rowbase + MB i + lane % MB for chunk kcol
  static constexpr int kFragReads = 1;  // LDS reads per fragment
  __device__ __forceinline__ u32x4 frag1(const char* st, int rowbase, int kcol, int i) const {
    const int row = rowbase + MB * i + (threadIdx.x & 63) % MB;
    return *(const u32x4*)(st + row * kStepBytes + ((kcol ^ swz(row)) << 4));
  }
  template <int NB>
  __device__ __forceinline__ void frag(const char* st, int rowbase, int kcol, u32x4 (&f)[NB]) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int row = rowbase + MB * i + lane % MB;
      f[i] = *(const u32x4*)(st + row * kStepBytes + ((kcol ^ swz(row)) << 4));
    }
  }
};

// K-contiguous operand in the blocked q layout (the rows of one tile, K = v): step ks is one 16 KiB
// block, row r of it at r * kStepBytes. Same LDS layout and fragments as OpK. Rows past the chunk
// hold values no output row uses (the grad_hidden rows past the chunk are dropped).
template <typename T>
struct OpKB : OpK<T> {
  using OpK<T>::BK;
  using OpK<T>::KV;
  using OpK<T>::RPI;
  const char* base;  // the tile's first block
  __device__ __forceinline__ void init(const T* blocks, int kmax_) {
    base = (const char*)blocks;
    this->kmax = kmax_;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kDmaPerOp; ++q) {
      const int row = RPI * (kDmaPerOp * wave + q) + lane / kChunks;
      this->kc[q] = (lane % kChunks) ^ OpK<T>::swz(row);
      this->rowoff[q] = (u32)(row * kStepBytes + this->kc[q] * 16);
    }
  }
  __device__ __forceinline__ void issue_one(int ks, u32 lds, int q) const {
    const int wave = threadIdx.x >> 6;
    const int k = ks * BK + this->kc[q] * KV;
    const i32x4 d = make_desc(base + (int64_t)ks * (TILE * kStepBytes), TILE * kStepBytes);
    dma16(d, k < this->kmax ? this->rowoff[q] : kOOB, lds + (kDmaPerOp * wave + q) * 1024);
  }
  __device__ __forceinline__ void issue(int ks, u32 lds) const {
#pragma unroll
    for (int q = 0; q < kDmaPerOp; ++q) issue_one(ks, lds, q);
  }
};

// MN-contiguous operand: a source row is one K index holding the tile's 256 M/N elements
// contiguously. In LDS a row keeps that layout (256 * sizeof(T) bytes), 16-byte chunk c stored at
// slot c ^ (kMnXor * (k & 3)). bf16 fragments come from two ds_read_b64_tr_b16: in each 16-lane group,
// lane j points at row k0 + j/4, columns nb + 4 (j % 4) .. +3, and lane i receives column nb + i of
// rows k0 .. k0+3 (gfx950 transpose read). The 16-lane groups differ in k0 (the lane's K chunk) and,
// for 32 x 32 blocks, in nb (columns 0-15 or 16-31 of the block). fp32 fragments are four
// ds_read_b32.
#ifndef FLCE_MN_XOR
#define FLCE_MN_XOR 4
#endif
constexpr int kMnXor = FLCE_MN_XOR;  // chunk XOR step per K row of an MN-contiguous operand in LDS
template <typename T>
struct OpMN {
  static constexpr int KV = 16 / sizeof(T), BK = kChunks * KV;
  static constexpr int ROWB = TILE * (int)sizeof(T);  // LDS bytes per K row
  static constexpr int CPR = ROWB / 16;               // chunks per row
  static constexpr int RPI = 64 / CPR;                // rows per DMA instruction (1 KiB)
  const char* p;       // element (k = 0, n = 0) of the tile
  int64_t ldb;         // source row stride in bytes
  int kvalid;          // valid K rows (also the end of this block's K range)
  u32 off[kDmaPerOp];  // byte offset of this lane's chunk within a stage's rows (kOOB if n invalid)
  __device__ __forceinline__ void init(const T* p_, int64_t ld, int kvalid_, int nvalid) {
    p = (const char*)p_;
    ldb = ld * (int64_t)sizeof(T);
    kvalid = kvalid_;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kDmaPerOp; ++q) {
      const int row = RPI * (kDmaPerOp * wave + q) + lane / CPR;
      const int c = (lane % CPR) ^ (kMnXor * (row & 3));
      off[q] = c * KV < nvalid ? (u32)(row * ldb + c * 16) : kOOB;
    }
  }
  // buffer descriptor of step ks: its BK source rows, rows past kvalid out of range
  __device__ __forceinline__ i32x4 step_desc(int ks) const {
    const int k0 = ks * BK;
    const int nrows = kvalid - k0 < 0 ? 0 : (kvalid - k0 > BK ? BK : kvalid - k0);
    return make_desc(p + (int64_t)k0 * ldb, (u32)nrows * (u32)ldb);
  }
  __device__ __forceinline__ void issue_one(int ks, u32 lds, int q) const {
    const int wave = threadIdx.x >> 6;
    dma16(step_desc(ks), off[q], lds + (kDmaPerOp * wave + q) * 1024);
  }
  __device__ __forceinline__ void issue(int ks, u32 lds) const {
    const int wave = threadIdx.x >> 6;
    const i32x4 desc = step_desc(ks);
#pragma unroll
    for (int q = 0; q < kDmaPerOp; ++q) dma16(desc, off[q], lds + (kDmaPerOp * wave + q) * 1024);
  }
  static constexpr int kFragReads = sizeof(T) == 2 ? 2 : 4;  // LDS reads per fragment
  __device__ __forceinline__ u32x4 frag1(const char* st, int colbase, int kcol, int i) const {
    const int lane = threadIdx.x & 63;
    u32x4 v;
    if constexpr (sizeof(T) == 2) {
      const int n = colbase + MB * i + (MB == 32 ? 16 * ((lane >> 4) & 1) : 0) + 4 * (lane & 3);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int k = 4 * (2 * kcol + r) + ((lane & 15) >> 2);  // kcol = frag_chunk(s, lane)
        const char* a = st + k * ROWB + (((n >> 3) ^ (kMnXor * (k & 3))) << 4) + ((n & 7) << 1);
        const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(size_t)lds_addr(a));
        const u32x2 w = __builtin_bit_cast(u32x2, t);
        v[2 * r] = w[0];
        v[2 * r + 1] = w[1];
      }
    } else {
      const int n = colbase + MB * i + lane % MB;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 4 * kcol + e;
        v[e] = *(const u32*)(st + k * ROWB + (((n >> 2) ^ (kMnXor * (k & 3))) << 4) + ((n & 3) << 2));
      }
    }
    return v;
  }
  template <int NB>
  __device__ __forceinline__ void frag(const char* st, int colbase, int kcol, u32x4 (&f)[NB]) const {
    const int lane = threadIdx.x & 63;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int n = colbase + MB * i + (MB == 32 ? 16 * ((lane >> 4) & 1) : 0) + 4 * (lane & 3);
        u32x4 v;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int k = 4 * (2 * kcol + r) + ((lane & 15) >> 2);  // kcol = frag_chunk(s, lane)
          const char* a = st + k * ROWB + (((n >> 3) ^ (kMnXor * (k & 3))) << 4) + ((n & 7) << 1);
          const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(size_t)lds_addr(a));
          const u32x2 w = __builtin_bit_cast(u32x2, t);
          v[2 * r] = w[0];
          v[2 * r + 1] = w[1];
        }
        f[i] = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int n = colbase + MB * i + lane % MB;
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 4 * kcol + e;
          v[e] = *(const u32*)(st + k * ROWB + (((n >> 2) ^ (kMnXor * (k & 3))) << 4) + ((n & 3) << 2));
        }
        f[i] = v;
      }
    }
  }
};

// MN-contiguous operand from the blocked q layout: q^T of one tile's 256 v, K = chunk rows. The
// 16-byte chunk c of K row k (v = v0 + c KV ..) lies in block (v0 + c KV) / kQB of k's tile of rows,
// at row k % 256. Same LDS layout and fragments as OpMN; K rows from kvalid on load zeros.
template <typename T>
struct OpMNB : OpMN<T> {
  using OpMN<T>::KV;
  using OpMN<T>::BK;
  using OpMN<T>::CPR;
  using OpMN<T>::RPI;
  static constexpr int QB = kQB<T>;
  static_assert(TILE % BK == 0, "a K step stays within one tile of rows");
  const char* base;     // tile of rows 0, the block of v0
  int64_t tstride;      // bytes per tile of rows
  int rowk[kDmaPerOp];  // the lane's K row within a step
  __device__ __forceinline__ void init(const T* q, int64_t nkv, int v0, int kvalid_) {
    base = (const char*)(q + (int64_t)(v0 / QB) * TILE * QB);
    tstride = nkv * TILE * kStepBytes;
    this->kvalid = kvalid_;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < kDmaPerOp; ++q) {
      const int row = RPI * (kDmaPerOp * wave + q) + lane / CPR;
      const int c = (lane % CPR) ^ (kMnXor * (row & 3));
      rowk[q] = row;
      this->off[q] = (u32)((c * KV / QB) * (TILE * kStepBytes) + row * kStepBytes + (c * KV % QB) * (int)sizeof(T));
    }
  }
  __device__ __forceinline__ void issue_one(int ks, u32 lds, int q) const {
    const int wave = threadIdx.x >> 6, k0 = ks * BK;
    const char* b = base + (int64_t)(k0 >> 8) * tstride + (int64_t)(k0 & (TILE - 1)) * kStepBytes;
    const i32x4 d = make_desc(b, (u32)(TILE / QB) * (TILE * kStepBytes));
    dma16(d, rowk[q] < this->kvalid - k0 ? this->off[q] : kOOB, lds + (kDmaPerOp * wave + q) * 1024);
  }
  __device__ __forceinline__ void issue(int ks, u32 lds) const {
#pragma unroll
    for (int q = 0; q < kDmaPerOp; ++q) issue_one(ks, lds, q);
  }
};

// ---- the MFMA tile core --------------------------------------------------------------------
// acc[i][j] is the MB x MB block (wave_m * WM + MB i, wave_n * WN + MB j) of the 256 x 256 tile, laid
// out as acc_row describes.
//
// K is consumed in steps of kStepBytes through a ring of kStages LDS stages filled by DMA, kStages-1
// steps ahead, into the slot the previous step read: issued at the step's start, or (FLCE_DMA_SPREAD)
// the first operand's loads within the step's first substep and the second operand's after its
// barrier. A step is kSub substeps of TBM x TBN MFMAs per wave; the fragments of substep s+1 are
// read while substep s runs, and those of the next step's substep 0 right after the step's single
// barrier, while its last substep runs. Prologue: DMA of the first kStages-1 steps (no waits).
template <class LA, class LB>
__device__ __forceinline__ void gemm_prologue(const LA& la, const LB& lb, int kb, char* smem) {
  const u32 lbase = lds_addr(smem);
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st) {
    la.issue(kb + st, lbase + st * kStageBytes);
    lb.issue(kb + st, lbase + st * kStageBytes + kOpBytes);
  }
}

template <typename T, class LA, class LB>
__device__ __forceinline__ void gemm_main(const LA& la, const LB& lb, int kb, int ke, char* smem,
                                          facc (&acc)[TBM][TBN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int i = 0; i < TBM; ++i)
#pragma unroll
    for (int j = 0; j < TBN; ++j)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.0f;
  const u32 lbase = lds_addr(smem);
  // any older vector-memory operations (loads and stores count alike) only make this wait stricter
  __builtin_amdgcn_s_waitcnt(vmcnt_only((kStages - 2) * kLoadsPerStage));
  asm volatile("s_barrier" ::: "memory");
  u32x4 fa[2][TBM], fb[2][TBN];
  la.frag(smem, wm * WM, frag_chunk(0, lane), fa[0]);
  lb.frag(smem + kOpBytes, wn * WN, frag_chunk(0, lane), fb[0]);
  for (int ks = kb; ks < ke; ++ks) {
    const int t = ks - kb;
    const char* st = smem + (t % kStages) * kStageBytes;
    // refill the slot the previous step read (every wave passed that step's barrier after its last
    // read of it); steps past the end load zeros
    const int nslot = (t + kStages - 1) % kStages;
    la.issue(ks + kStages - 1, lbase + nslot * kStageBytes);
    lb.issue(ks + kStages - 1, lbase + nslot * kStageBytes + kOpBytes);
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      if (s + 1 < kSub) {
        la.frag(st, wm * WM, frag_chunk(s + 1, lane), fa[(s + 1) & 1]);
        lb.frag(st + kOpBytes, wn * WN, frag_chunk(s + 1, lane), fb[(s + 1) & 1]);
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_only((kStages - 2) * kLoadsPerStage));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const char* nx = smem + ((t + 1) % kStages) * kStageBytes;
        la.frag(nx, wm * WM, frag_chunk(0, lane), fa[(s + 1) & 1]);
        lb.frag(nx + kOpBytes, wn * WN, frag_chunk(0, lane), fb[(s + 1) & 1]);
      }
#pragma unroll
      for (int i = 0; i < TBM; ++i)
#pragma unroll
        for (int j = 0; j < TBN; ++j) mma(acc[i][j], fa[s & 1][i], fb[s & 1][j], (T*)nullptr);
    }
  }
  // the DMA of the steps past the end must land before the LDS is reused or the block ends; the
  // barrier makes every wave finish its reads before a following prologue refills the ring
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The same pipeline with the step loop unrolled by kStages: stage slots and LDS offsets are
// compile-time constants and the loop body has no exits. The step count is rounded up to a multiple
// of kStages; steps past ke load zeros (out of range) and add nothing. With RPM > 0 the scheduler
// places RPM fragment reads after each MFMA until the substep's reads are placed, so LDS requests
// trickle instead of queueing behind the DMA writes, and no read is left after the substep's last
// MFMA (where the step's barrier, or the next substep's first MFMA, would wait for it in full).
template <typename T, int RPM, class LA, class LB>
__device__ __forceinline__ void gemm_main_u(const LA& la, const LB& lb, int kb, int ke, char* smem,
                                            facc (&acc)[TBM][TBN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int i = 0; i < TBM; ++i)
#pragma unroll
    for (int j = 0; j < TBN; ++j)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.0f;
  const u32 lbase = lds_addr(smem);
  __builtin_amdgcn_s_waitcnt(vmcnt_only((kStages - 2) * kLoadsPerStage));
  asm volatile("s_barrier" ::: "memory");
  u32x4 fa[2][TBM], fb[2][TBN];
  la.frag(smem, wm * WM, frag_chunk(0, lane), fa[0]);
  lb.frag(smem + kOpBytes, wn * WN, frag_chunk(0, lane), fb[0]);
  for (int ks0 = kb; ks0 < ke; ks0 += kStages) {
#pragma unroll
    for (int t = 0; t < kStages; ++t) {
      const int ks = ks0 + t;
      const char* st = smem + t * kStageBytes;
      const int nslot = (t + kStages - 1) % kStages;
      const u32 dst = lbase + nslot * kStageBytes;
      if constexpr (!kSpread) {
        la.issue(ks + kStages - 1, dst);
        lb.issue(ks + kStages - 1, dst + kOpBytes);
      }
#pragma unroll
      for (int s = 0; s < kSub; ++s) {
        if (s + 1 < kSub) {
          la.frag(st, wm * WM, frag_chunk(s + 1, lane), fa[(s + 1) & 1]);
          lb.frag(st + kOpBytes, wn * WN, frag_chunk(s + 1, lane), fb[(s + 1) & 1]);
        } else {
          // the next step's stage must have landed: with the second operand's loads of this step
          // still to come, only the steps after it and this step's first-operand loads may remain
          __builtin_amdgcn_s_waitcnt(vmcnt_only(kSpread ? (kStages - 3) * kLoadsPerStage + kDmaPerOp
                                                        : (kStages - 2) * kLoadsPerStage));
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          const char* nx = smem + ((t + 1) % kStages) * kStageBytes;
          la.frag(nx, wm * WM, frag_chunk(0, lane), fa[(s + 1) & 1]);
          lb.frag(nx + kOpBytes, wn * WN, frag_chunk(0, lane), fb[(s + 1) & 1]);
        }
#pragma unroll
        for (int i = 0; i < TBM; ++i)
#pragma unroll
          for (int j = 0; j < TBN; ++j) {
            mma(acc[i][j], fa[s & 1][i], fb[s & 1][j], (T*)nullptr);
            if constexpr (kSpread) {
              // slot nslot was last read before the previous step's barrier
              if (s == 0 && i * TBN + j < kDmaPerOp) la.issue_one(ks + kStages - 1, dst, i * TBN + j);
              if (s == kSub - 1 && i * TBN + j < kDmaPerOp) lb.issue_one(ks + kStages - 1, dst + kOpBytes, i * TBN + j);
            }
          }
        if constexpr (RPM > 0) {
          constexpr int nr = TBM * LA::kFragReads + TBN * LB::kFragReads, nm = TBM * TBN;
          constexpr int gf = nr / RPM < nm ? nr / RPM : nm;               // MFMAs followed by RPM reads
          constexpr int gp = gf < nm && gf * RPM < nr && nr - gf * RPM < RPM ? 1 : 0;  // one followed by fewer
          constexpr int placed = gf * RPM + (gp ? nr - gf * RPM : 0);
#pragma unroll
          for (int q = 0; q < gf; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);  // RPM LDS reads
          }
          if constexpr (gp) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, nr - gf * RPM, 0);
          }
          if constexpr (nm > gf + gp) __builtin_amdgcn_sched_group_barrier(0x008, nm - gf - gp, 0);
          if constexpr (nr > placed) __builtin_amdgcn_sched_group_barrier(0x100, nr - placed, 0);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The unrolled pipeline with an explicit instruction order: each MFMA of a substep is followed by
// the fragment reads assigned to it and, in the spread placement, by one DMA load, and nothing is
// scheduled across these groups. The next substep's fragments are read in the order its MFMAs use
// them (B_0, A_0, B_1, A_1, ..., then the remaining A), up to RPM LDS instructions after each
// MFMA, so the last read of a substep is issued several MFMAs before the barrier that waits for it.
template <int RPM, class LA, class LB>
struct XOrder {
  static constexpr int NFR = TBM + TBN, NM = TBM * TBN;
  static constexpr bool is_b(int f) { return f < 2 * TBN ? (f % 2 == 0) : false; }
  static constexpr int idx(int f) { return f < 2 * TBN ? f / 2 : f - TBN; }
  static constexpr int reads(int f) { return is_b(f) ? LB::kFragReads : LA::kFragReads; }
  static constexpr int group(int f) {
    int c = 0;
    for (int g = 0; g < f; ++g) c += reads(g);
    return c / RPM < NM - 1 ? c / RPM : NM - 1;
  }
};
template <typename T, int RPM, class LA, class LB>
__device__ __forceinline__ void gemm_main_x(const LA& la, const LB& lb, int kb, int ke, char* smem,
                                            facc (&acc)[TBM][TBN]) {
  using O = XOrder<RPM, LA, LB>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int i = 0; i < TBM; ++i)
#pragma unroll
    for (int j = 0; j < TBN; ++j)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.0f;
  const u32 lbase = lds_addr(smem);
  __builtin_amdgcn_s_waitcnt(vmcnt_only((kStages - 2) * kLoadsPerStage));
  asm volatile("s_barrier" ::: "memory");
  u32x4 fa[2][TBM], fb[2][TBN];
  la.frag(smem, wm * WM, frag_chunk(0, lane), fa[0]);
  lb.frag(smem + kOpBytes, wn * WN, frag_chunk(0, lane), fb[0]);
  for (int ks0 = kb; ks0 < ke; ks0 += kStages) {
#pragma unroll
    for (int t = 0; t < kStages; ++t) {
      const int ks = ks0 + t;
      const char* st = smem + t * kStageBytes;
      const int nslot = (t + kStages - 1) % kStages;
      const u32 dst = lbase + nslot * kStageBytes;
      if constexpr (!kSpread) {
        la.issue(ks + kStages - 1, dst);
        lb.issue(ks + kStages - 1, dst + kOpBytes);
      }
#pragma unroll
      for (int s = 0; s < kSub; ++s) {
        const char* src = st;
        int kcol = frag_chunk(s + 1, lane);
        if (s + 1 == kSub) {
          __builtin_amdgcn_s_waitcnt(vmcnt_only(kSpread ? (kStages - 3) * kLoadsPerStage + kDmaPerOp
                                                        : (kStages - 2) * kLoadsPerStage));
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          src = smem + ((t + 1) % kStages) * kStageBytes;
          kcol = frag_chunk(0, lane);
        }
        const int cb = s & 1, rb = (s + 1) & 1;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < O::NM; ++q) {
          mma(acc[q / TBN][q % TBN], fa[cb][q / TBN], fb[cb][q % TBN], (T*)nullptr);
#pragma unroll
          for (int f = 0; f < O::NFR; ++f) {
            if (O::group(f) == q) {
              if (O::is_b(f))
                fb[rb][O::idx(f)] = lb.frag1(src + kOpBytes, wn * WN, kcol, O::idx(f));
              else
                fa[rb][O::idx(f)] = la.frag1(src, wm * WM, kcol, O::idx(f));
            }
          }
          if constexpr (kSpread) {
            // slot nslot was last read before the previous step's barrier
#pragma unroll
            for (int d = 0; d < kDmaPerOp; ++d) {
              if (q == FLCE_DMA_FIRST + d * FLCE_DMA_STRIDE) {
                if (s == 0) la.issue_one(ks + kStages - 1, dst, d);
                if (s == kSub - 1) lb.issue_one(ks + kStages - 1, dst + kOpBytes, d);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The pipeline for 16 x 16 blocks: one MFMA covers the step's 32 K per block, so a step is split in
// two substeps over the M blocks (the wave's first TBM/2 row blocks, then the others), each with all
// TBN column blocks. The A fragments of the second half are read while the first half runs; at the
// step's barrier the next step's first-half A fragments and all its B fragments are read, into the
// other B buffer, while the second half runs. Unrolled by the ring depth (even), so buffer indices
// and stage offsets are constants.
template <typename T, bool INTERLEAVE, class LA, class LB>
__device__ __forceinline__ void gemm_main16(const LA& la, const LB& lb, int kb, int ke, char* smem,
                                            facc (&acc)[TBM][TBN]) {
  static_assert(MB == 16 && kChunks == 4 && kStages % 2 == 0, "16 x 16 blocks: 64-byte steps, even ring");
  constexpr int HM = TBM / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1, kq = frag_chunk(0, lane);
#pragma unroll
  for (int i = 0; i < TBM; ++i)
#pragma unroll
    for (int j = 0; j < TBN; ++j)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.0f;
  const u32 lbase = lds_addr(smem);
  __builtin_amdgcn_s_waitcnt(vmcnt_only((kStages - 2) * kLoadsPerStage));
  asm volatile("s_barrier" ::: "memory");
  u32x4 fa[2][HM], fb[2][TBN];
  la.frag(smem, wm * WM, kq, fa[0]);
  lb.frag(smem + kOpBytes, wn * WN, kq, fb[0]);
  for (int ks0 = kb; ks0 < ke; ks0 += kStages) {
#pragma unroll
    for (int t = 0; t < kStages; ++t) {
      const int ks = ks0 + t;
      const char* st = smem + t * kStageBytes;
      const int nslot = (t + kStages - 1) % kStages;
      la.issue(ks + kStages - 1, lbase + nslot * kStageBytes);
      lb.issue(ks + kStages - 1, lbase + nslot * kStageBytes + kOpBytes);
      // substep 0: the first HM row blocks; the second half's A fragments are read meanwhile
      la.frag(st, wm * WM + HM * MB, kq, fa[1]);
#pragma unroll
      for (int i = 0; i < HM; ++i)
#pragma unroll
        for (int j = 0; j < TBN; ++j) mma(acc[i][j], fa[0][i], fb[t & 1][j], (T*)nullptr);
      if constexpr (INTERLEAVE) {
        constexpr int nr = HM * LA::kFragReads, nm = HM * TBN, np = nr < nm ? nr : nm;
#pragma unroll
        for (int q = 0; q < np; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (nm > np) __builtin_amdgcn_sched_group_barrier(0x008, nm - np, 0);
        if constexpr (nr > np) __builtin_amdgcn_sched_group_barrier(0x100, nr - np, 0);
      }
      // substep 1: the second half; after the barrier the next step's fragments are read meanwhile
      __builtin_amdgcn_s_waitcnt(vmcnt_only((kStages - 2) * kLoadsPerStage));
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const char* nx = smem + ((t + 1) % kStages) * kStageBytes;
      la.frag(nx, wm * WM, kq, fa[0]);
      lb.frag(nx + kOpBytes, wn * WN, kq, fb[(t + 1) & 1]);
#pragma unroll
      for (int i = 0; i < HM; ++i)
#pragma unroll
        for (int j = 0; j < TBN; ++j) mma(acc[HM + i][j], fa[1][i], fb[t & 1][j], (T*)nullptr);
      if constexpr (INTERLEAVE) {
        constexpr int nr = HM * LA::kFragReads + TBN * LB::kFragReads, nm = HM * TBN;
        constexpr int np = nr < nm ? nr : nm;
#pragma unroll
        for (int q = 0; q < np; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (nm > np) __builtin_amdgcn_sched_group_barrier(0x008, nm - np, 0);
        if constexpr (nr > np) __builtin_amdgcn_sched_group_barrier(0x100, nr - np, 0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Main-loop schedules of the GEMM core: rolled, unrolled, and unrolled with one or two fragment
// reads placed after each MFMA.
enum Sched { kRolled = 0, kUnrolled = 1, kInterleaved = 2, kInterleaved2 = 3, kExplicit1 = 4, kExplicit2 = 5,
             kExplicit3 = 6 };
// The main loop of the schedule SCHED, after a prologue issued by the caller.
template <typename T, int SCHED, class LA, class LB>
__device__ __forceinline__ void gemm_main_sched(const LA& la, const LB& lb, int kb, int ke, char* smem,
                                                facc (&acc)[TBM][TBN]) {
  if constexpr (MB == 16)
    gemm_main16<T, SCHED >= kInterleaved && sizeof(T) == 2>(la, lb, kb, ke, smem, acc);
  else if constexpr (SCHED == kRolled)
    gemm_main<T>(la, lb, kb, ke, smem, acc);
  else if constexpr (SCHED >= kExplicit1)
    gemm_main_x<T, SCHED - kExplicit1 + 1>(la, lb, kb, ke, smem, acc);
  else
    gemm_main_u<T, SCHED == kInterleaved2 ? 2 : SCHED == kInterleaved ? 1 : 0>(la, lb, kb, ke, smem, acc);
}
template <typename T, int SCHED, class LA, class LB>
__device__ __forceinline__ void gemm_core(const LA& la, const LB& lb, int kb, int ke, char* smem,
                                          facc (&acc)[TBM][TBN]) {
  if (kb >= ke) {
#pragma unroll
    for (int i = 0; i < TBM; ++i)
#pragma unroll
      for (int j = 0; j < TBN; ++j)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.0f;
    return;
  }
  gemm_prologue(la, lb, kb, smem);
  gemm_main_sched<T, SCHED>(la, lb, kb, ke, smem, acc);
}

// ---- kernel arguments ------------------------------------------------------------------------
struct FwdArgs {
  const void* XT;     // [H][ldt]: the chunk of hidden, transposed
  int64_t ldt;
  const void* W;
  void* ws;
  float* seg_m;
  float* seg_s;
  const int* y;       // chunk row 0: label or -1
  float* s_label;     // chunk row 0
  const float* cref;  // chunk row 0: the reference c of each row (q = exp(s - c) ...)
  int64_t H, V, V_pad;  // V columns of W starting at W's row 0 (a slice of the vocabulary: V = slice width)
  int nseg, rows;
  int yoff;           // vocabulary index of W's row 0: labels are taken relative to it
  float softcap;
};

struct DxArgs {
  const void* W;
  const void* ws;     // q of the chunk, blocked layout (q_index) with V_pad / kQB blocks per tile of rows
  const float* fscale;  // chunk row 0: the per-row factor f of dZ = f q (applied to the output rows)
  void* out;          // grad_hidden (splits == 1): row r of the call starts at element gmap(r)
  RowMap gmap;
  int64_t row0;       // call row of chunk row 0
  float* part;        // [splits][rows][H] fp32 partials (splits > 1, or part_out)
  int64_t H, V, V_pad;
  int rows, splits, ksteps_per_split, accumulate;
  int part_out;       // 1: write the fp32 [rows][H] partials even with one split
  int part_acc;       // 1: add to the fp32 partials instead of writing them (one split)
};

struct DwArgs {
  const void* X;      // hidden_f = f hidden of the chunk, [rows][H]
  const void* ws;     // q of the chunk, blocked layout (q_index) with V_pad / kQB blocks per tile of rows
  float* dW;
  int64_t H, V, V_pad;
  int rows, accumulate;
  // the last wave's tiles split along K: tiles [full, mt * nt) of the grouped order are computed as
  // tail_splits partial sums each, written to tail_part and added by k_dw_tail
  int full, tail_splits;
  float* tail_part;   // [tiles - full][tail_splits][256][256]
};

// Tile-row group sizes of the grouped tile order (measured on MI355X at the Llama-3-8B head). Each
// XCD runs 32 blocks at once; for the products with M = V (logits, grad_W) a group of 4 V-tiles
// swept over the tiles of the small operand (a chunk of hidden) halves the small operand's re-reads
// from the last-level cache against groups of 2, while the large operand's panels (W or dZ) stay in
// the XCD's L2 for the round that uses them.
#ifndef FLCE_GROUP_FWD
#define FLCE_GROUP_FWD 4
#endif
#ifndef FLCE_GROUP_DX
#define FLCE_GROUP_DX 4
#endif
#ifndef FLCE_GROUP_DW
#define FLCE_GROUP_DW 4
#endif
// Main-loop schedule per product (Sched: 0 rolled, 1 unrolled, 2 and 3 unrolled with one or two
// fragment reads placed after each MFMA by the scheduler, 4 to 6 the explicit order with up to 1 to 3
// LDS reads after each MFMA). On MI355X the explicit order with two reads per MFMA and the spread DMA
// placement measured best for all three products at the Llama-3-8B and GPT-2 heads.
#ifndef FLCE_SCHED_FWD
#define FLCE_SCHED_FWD 5
#endif
#ifndef FLCE_SCHED_DX
#define FLCE_SCHED_DX 5
#endif
#ifndef FLCE_SCHED_DW
#define FLCE_SCHED_DW (FLCE_MFMA == 16 ? 1 : 5)
#endif
constexpr int kSchedFwd = FLCE_SCHED_FWD;
constexpr int kSchedDx = FLCE_SCHED_DX;
constexpr int kSchedDw = FLCE_SCHED_DW;
constexpr int kGroupFwd = FLCE_GROUP_FWD;
constexpr int kGroupDx = FLCE_GROUP_DX;
constexpr int kGroupDw = FLCE_GROUP_DW;

// ---- forward: logits tile + softcap + segment statistics + q store -------------------------
// Epilogue of one wave's 128 (v) x 128 (chunk row) quarter, specialised on the softcap (CAP) and on
// whether the quarter crosses V (EDGE): the common case has no per-element masking at all. For each
// 32-row block j, each lane holds column c (a chunk row) and 64 v values; the two lanes c and c+32
// hold the two halves of the wave's 128-wide segment of row c.
// Labels of this lane's chunk rows (range-checked loads; -1 past the chunk).
__device__ __forceinline__ void fwd_labels(const FwdArgs& a, int c0, int (&ylab)[TBN]) {
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) >> 1;
  const rsrc_t ry = make_rsrc(a.y, (int64_t)a.rows * 4);
#pragma unroll
  for (int j = 0; j < TBN; ++j) {
    const int c = c0 + wn * WN + MB * j + lane % MB;
    const int yv = __builtin_amdgcn_raw_buffer_load_b32(ry, c * 4, 0, 0);
    ylab[j] = c < a.rows && yv >= 0 ? yv - a.yoff : -1;
  }
}

// q tiles of 16-bit values are staged per wave through the (then idle) LDS ring: each wave stages
// half of one column block at a time, the MB rows of half its WM v values (one 128-byte line per row,
// 16-byte chunks XOR-swizzled by the row), in an area of its own in the ring's last slot, and writes
// them out itself as soon as the half is complete, as 64-byte pieces that with those of the
// neighbouring rows make 2 KiB runs of the blocked layout. No block barrier is involved and the
// stores of one half overlap the arithmetic of the next. (The accumulator layout alone gives 8-byte
// pieces of 32 rows per store.) Measured on MI355X against staging the whole tile through the ring
// (one barrier, then all threads store): logits GEMM 3.33 against 3.37 ms at the Llama-3-8B head,
// 1.30 against 1.36 ms at the GPT-2 head.
template <typename T>
constexpr bool kStageQ = sizeof(typename Traits<T>::S) == 2;
constexpr int kQwRow = WM;                  // bytes per staged row: WM / 2 16-bit values
constexpr int kQwBytes = MB * kQwRow;       // per wave and half column block
constexpr int kQwBase = (kStages - 1) * kStageBytes;
static_assert(kQwBase + NW * kQwBytes <= kStages * kStageBytes, "per-wave q staging fits the ring's last slot");
__device__ __forceinline__ u32 qwlds(int cr, int vl) {  // q(row cr of the column block, v vl of the half)
  return (u32)(cr * kQwRow + (((vl >> 3) ^ (cr & (kQwRow / 16 - 1))) << 4) + ((vl & 7) << 1));
}

// QONLY: store q only (slices of the recompute mode), no statistics or label logits.
// For each column block j, a lane holds column c (a chunk row) and WM / (64 / MB) of the wave's 128
// v values of that row: the 64 / MB lanes that share c (c + k MB) hold the rest, and the row's
// segment statistics are combined across them with lane exchanges.
template <typename T, bool CAP, bool EDGE, bool STORE_Q, bool QONLY, int J0, int JG>
__device__ __forceinline__ void fwd_epilogue_part(const FwdArgs& a, facc (&acc)[TBM][TBN], int v0, int c0,
                                                  const int (&ylab)[TBN], char* smem) {
  using S = typename Traits<T>::S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  const int vw = v0 + wm * WM, seg = vw / kSeg, col = lane % MB, vl0 = acc_row(0, lane);
  const float cap = a.softcap, icap = CAP ? 1.0f / cap : 0.0f;
  // references of the lane's rows (0 past the chunk), consumed in phase 3
  float cr[TBN];
  {
    const rsrc_t rc = make_rsrc(a.cref, (int64_t)a.rows * 4);
#pragma unroll
    for (int j = J0; j < J0 + JG; ++j) cr[j] = bload_f32(rc, (u32)(c0 + wn * WN + MB * j + col) * 4, 0);
  }
  // Column blocks J0 .. J0+JG-1. They are independent; each phase runs over all of them so that the
  // wave has independent work (and the cross-lane exchanges are in flight together).
  // Phase 1: softcap in place and the maxima (one chain per row block i).
  float mx[TBN] = {};
#pragma unroll
  for (int j = J0; j < J0 + JG; ++j) {
    float m4[TBM];
#pragma unroll
    for (int i = 0; i < TBM; ++i) {
      m4[i] = kNegInf;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float s = acc[i][j][r];
        if constexpr (CAP) {
          s = cap * tanh_via_exp(s * icap);
          acc[i][j][r] = s;
        }
        if constexpr (EDGE) {
          const int v = vw + MB * i + acc_row(r, lane);
          s = v < a.V ? s : kNegInf;
        }
        m4[i] = fmaxf(m4[i], s);
      }
    }
    float m = m4[0];
#pragma unroll
    for (int i = 1; i < TBM; ++i) m = fmaxf(m, m4[i]);
    mx[j] = m;
  }
  // Phase 2: the lanes c, c + MB, ... hold the parts of a row's 128-wide segment.
#pragma unroll
  for (int x = MB; x < 64; x *= 2) {
    float o[TBN];
#pragma unroll
    for (int j = J0; j < J0 + JG; ++j) o[j] = __shfl_xor(mx[j], x);
#pragma unroll
    for (int j = J0; j < J0 + JG; ++j) mx[j] = fmaxf(mx[j], o[j]);
  }
  // Phase 3: the segment's reference r = max(c, segment max - kRefSpan), so that every e = exp(s - r)
  // is at most exp(kRefSpan) (r = c unless the label logit lies more than kRefSpan below the segment
  // maximum; k_lse rescales such rows), the sums of e, and q = e (times the softcap derivative) to the
  // workspace. Rows that do not count have c = -inf, hence r = segment max - kRefSpan.
  // q tile: rows c0.. of the chunk, columns v0 .. v0+255 < V_pad, in the tile of rows c0 / 256 of the
  // blocked layout; rows past the chunk are not stored
  constexpr int QB = kQB<S>;
  const int64_t nkv = a.V_pad / QB;
  const rsrc_t rq = make_rsrc((S*)a.ws + (int64_t)(c0 / TILE) * nkv * TILE * QB, nkv * TILE * kStepBytes);
  const auto qoff = [&](int cl, int v) -> u32 {  // byte offset of q(c0 + cl, v) in that tile of rows
    return c0 + cl < a.rows ? (u32)(((v / QB) * TILE + cl) * QB + v % QB) * (u32)sizeof(S) : kOOB;
  };
  float sum[TBN] = {}, rf[TBN];
#pragma unroll
  for (int j = J0; j < J0 + JG; ++j) {
    const int c = c0 + wn * WN + MB * j + col;
    // (a segment wholly past V has no maximum; its e are masked to 0 and its statistics record -inf)
    rf[j] = mx[j] == kNegInf ? 0.0f : fmaxf(cr[j], mx[j] - kRefSpan);
    const float msl = -rf[j] * kLog2e;
    // the lane's offset of q(c, v0 + wm WM + vl0) for the unstaged (fp32) stores, or past the range
    const u32 qlane = c < a.rows ? qoff(c - c0, v0 + wm * WM + vl0) : kOOB;
    (void)qlane;
    float sum4[TBM];
#pragma unroll
    for (int i = 0; i < TBM; ++i) {
      sum4[i] = 0.0f;
#pragma unroll
      for (int g = 0; g < NR / 4; ++g) {
        float q[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float s = acc[i][j][4 * g + rr];
          float e = ex2(fmaf(s, kLog2e, msl));  // 2^((s - r) log2 e)
          if constexpr (EDGE) {
            const int v = vw + MB * i + acc_row(4 * g + rr, lane);
            e = v < a.V ? e : 0.0f;
          }
          sum4[i] += e;
          if constexpr (CAP) {
            const float t = s * icap;
            q[rr] = e * (1.0f - t * t);
          } else {
            q[rr] = e;
          }
        }
        // registers 4g .. 4g+3 are rows acc_row(4g) .. +3 of block i: four consecutive v
        const int vblk = MB * i + acc_row(4 * g, 0);
        if constexpr (!STORE_Q) {
        } else if constexpr (kStageQ<T>) {
          *(u32x2*)(smem + kQwBase + wave * kQwBytes + qwlds(col, vl0 + vblk - (i / (TBM / 2)) * (WM / 2))) =
              pack4_bf16(q[0], q[1], q[2], q[3]);
        } else {
          // v = v0 + wm WM + vl0 + vblk: the lane's part vl0 (< 16) and vblk % kQB (at most 8) stay
          // within one block, so the offset is the lane's qlane plus a constant per (i, g). The sum is
          // selected per lane: with the constant in the scalar offset register instead, these 16-byte
          // stores, whose data registers the next instruction rewrites, stored wrong data in some lanes
          // on MI355X (no wait state is inserted for that form).
          const u32 o = c < a.rows ? qlane + (u32)(((vblk / QB) * TILE * QB + vblk % QB) * (int)sizeof(S)) : kOOB;
          bstore_b128(rq, o, __builtin_bit_cast(u32x4, f32x4{q[0], q[1], q[2], q[3]}));
        }
      }
      if constexpr (STORE_Q && kStageQ<T>) {
        if (i % (TBM / 2) == TBM / 2 - 1) {
          // half h of the wave's v values for the MB rows of column block j, one line per row
          const int h = i / (TBM / 2);
          const char* wb = smem + kQwBase + wave * kQwBytes;
          constexpr int kCh = kQwRow / 16, kRowsPerInst = 64 / kCh;
          const int ch = lane % kCh;
#pragma unroll
          for (int r0 = 0; r0 < MB; r0 += kRowsPerInst) {
            const int cr = r0 + lane / kCh;
            const u32x4 v = *(const u32x4*)(wb + cr * kQwRow + ((ch ^ (cr & (kCh - 1))) << 4));
            const int cl = wn * WN + MB * j + cr;  // chunk row within the tile
            bstore_b128(rq, qoff(cl, v0 + wm * WM + h * (WM / 2) + ch * 8), v);
          }
        }
      }
    }
    float t = sum4[0];
#pragma unroll
    for (int i = 1; i < TBM; ++i) t += sum4[i];
    sum[j] = t;
  }
  // Phases 4 and 5 (not for vocabulary slices, whose statistics exist already).
  if constexpr (QONLY) return;
  // Phase 4: segment statistics of the tile's rows.
#pragma unroll
  for (int x = MB; x < 64; x *= 2) {
    float o[TBN];
#pragma unroll
    for (int j = J0; j < J0 + JG; ++j) o[j] = __shfl_xor(sum[j], x);
#pragma unroll
    for (int j = J0; j < J0 + JG; ++j) sum[j] += o[j];
  }
#pragma unroll
  for (int j = J0; j < J0 + JG; ++j) {
    const int c = c0 + wn * WN + MB * j + col;
    if (lane < MB && c < a.rows) {
      a.seg_m[(int64_t)c * a.nseg + seg] = mx[j] == kNegInf ? kNegInf : rf[j];
      a.seg_s[(int64_t)c * a.nseg + seg] = sum[j];
    }
  }
  // Phase 5: the label logit of row c, taken from the same fp32 value that entered the row
  // statistics; exactly one lane of the whole grid holds (v = y_c, c).
#pragma unroll
  for (int j = J0; j < J0 + JG; ++j) {
    const unsigned rel = (unsigned)(ylab[j] - vw);
    // for the lane that holds it: block i = rel / MB, and within the block row rb = rel % MB, which
    // is acc_row(rsel, lane) for one lane group and register
    const int rb = (int)(rel % MB);
    int isel, rsel;
    bool mine;
    if constexpr (MB == 32) {
      mine = rel < (unsigned)WM && ((rb >> 2) & 1) == (lane >> 5);
      rsel = 4 * (rb >> 3) + (rb & 3);
    } else {
      mine = rel < (unsigned)WM && (rb >> 2) == (lane >> 4);
      rsel = rb & 3;
    }
    isel = (int)(rel / MB);
    if (__any(mine)) {
      float sy = 0.0f;
#pragma unroll
      for (int i = 0; i < TBM; ++i) {
        float t = acc[i][j][0];
#pragma unroll
        for (int r = 1; r < NR; ++r) t = rsel == r ? acc[i][j][r] : t;
        sy = isel == i ? t : sy;
      }
      if (mine) {
        const int c = c0 + wn * WN + MB * j + col;
        a.s_label[c] = sy;
      }
    }
  }
}

template <typename T, bool CAP, bool EDGE, bool STORE_Q, bool QONLY, int J0 = 0>
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& a, facc (&acc)[TBM][TBN], int v0, int c0,
                                             const int (&ylab)[TBN], char* smem) {
  // two column blocks at a time: enough independent work, few enough live values to stay in registers
  if constexpr (J0 < TBN) {
    constexpr int JG = TBN - J0 < 2 ? TBN - J0 : 2;
    fwd_epilogue_part<T, CAP, EDGE, STORE_Q, QONLY, J0, JG>(a, acc, v0, c0, ylab, smem);
    fwd_epilogue<T, CAP, EDGE, STORE_Q, QONLY, J0 + JG>(a, acc, v0, c0, ylab, smem);
  }
}

template <typename T>
__device__ __forceinline__ void fwd_loaders(const FwdArgs& a, int v0, int c0, OpK<T>& la, OpMN<T>& lb) {
  la.init((const T*)a.W + (int64_t)v0 * a.H, a.H, (int)min<int64_t>(TILE, a.V - v0), (int)a.H);  // W rows v0..
  lb.init((const T*)a.XT + c0, a.ldt, (int)a.H, min(TILE, a.rows - c0));  // hidden^T: rows h, columns c0..
}
// One 256 x 256 tile of the logits product and its epilogue. STORE_Q = false is the forward-only
// path: the row statistics and label logits are produced, the q tile is not stored. QONLY: q only.
template <typename T, bool STORE_Q, bool QONLY>
__device__ __forceinline__ void fwd_tile(const FwdArgs& a, int v0, int c0, char* smem) {
  OpK<T> la;
  OpMN<T> lb;
  fwd_loaders<T>(a, v0, c0, la, lb);
  // the labels are loaded before the main loop, whose first wait on the operand loads covers them
  int ylab[TBN];
  fwd_labels(a, c0, ylab);
  facc acc[TBM][TBN];
  const int nk = (int)((a.H + OpK<T>::BK - 1) / OpK<T>::BK);
  static_assert(OpK<T>::BK == OpMN<T>::BK, "operands step through K together");
  gemm_core<T, kSchedFwd>(la, lb, 0, nk, smem, acc);

  // wave-uniform selection of the specialised epilogue
  const bool edge = v0 + (((int)threadIdx.x >> 6) & 1) * WM + WM > a.V;
  if (a.softcap > 0.0f) {
    if (edge)
      fwd_epilogue<T, true, true, STORE_Q, QONLY>(a, acc, v0, c0, ylab, smem);
    else
      fwd_epilogue<T, true, false, STORE_Q, QONLY>(a, acc, v0, c0, ylab, smem);
  } else {
    if (edge)
      fwd_epilogue<T, false, true, STORE_Q, QONLY>(a, acc, v0, c0, ylab, smem);
    else
      fwd_epilogue<T, false, false, STORE_Q, QONLY>(a, acc, v0, c0, ylab, smem);
  }
}

template <typename T, bool STORE_Q, bool QONLY>
__global__ __launch_bounds__(NTHR) void k_fwd(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kStages * kStageBytes];
  const int mt = (int)(a.V_pad / TILE), nt = (a.rows + TILE - 1) / TILE;
  int tm, tn;
  grouped(xcd_remap(blockIdx.x, gridDim.x), mt, nt, kGroupFwd, tm, tn);
  fwd_tile<T, STORE_Q, QONLY>(a, tm * TILE, tn * TILE, smem);
}

// ---- grad_hidden = f . (q . W) -------------------------------------------------------------------
// The fp32 tile goes through the (then idle) LDS ring in passes of kDxPassRows rows and leaves as
// 16-byte pieces of whole caller rows: each row is multiplied by its factor f, placed by the row map
// (sequences with strides, shifted labels), and with `accumulate` added to what the row holds (one
// rounding to the output type, after the add). Pass p stages row blocks 2p and 2p+1 of every wave (tile rows
// wm * WM + 64 p .. + 63), so the accumulators of a pass are dead before its read-out.
constexpr int kDxRowBytes = TILE * 4;
constexpr int kDxPassRows = WM;
static_assert(kDxPassRows * kDxRowBytes <= kStages * kStageBytes, "a pass fits the LDS ring");
static_assert(TBM % (TILE / kDxPassRows) == 0 && kDxPassRows == 2 * MB * (TBM / (TILE / kDxPassRows)),
              "a pass stages the same number of row blocks of each of the two wave-rows");
template <typename T>
__device__ __forceinline__ void dx_store_tile(const DxArgs& a, const facc (&acc)[TBM][TBN], int c0, int h0,
                                              int vrows, char* smem) {
  constexpr int OV = 16 / (int)sizeof(T);  // output elements per 16-byte store
  constexpr int TPR = TILE / OV;           // threads per row
  constexpr int RPI = NTHR / TPR;          // rows per read-out iteration
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  const int ch = (int)threadIdx.x % TPR, h = h0 + ch * OV;
  constexpr int kBlocksPerPass = TBM / (TILE / kDxPassRows);  // row blocks of a wave per pass
  constexpr int kWaveRows = MB * kBlocksPerPass;              // rows of a wave-row per pass (64)
#pragma unroll
  for (int pass = 0; pass < TILE / kDxPassRows; ++pass) {
#pragma unroll
    for (int ib = 0; ib < kBlocksPerPass; ++ib) {
      const int i = pass * kBlocksPerPass + ib;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int rl = wm * kWaveRows + MB * ib + acc_row(r, lane);
#pragma unroll
        for (int j = 0; j < TBN; ++j) {
          const int cl = wn * WN + MB * j + lane % MB;
          *(float*)(smem + rl * kDxRowBytes + cl * 4) = acc[i][j][r];
        }
      }
    }
    __syncthreads();
    for (int rl = (int)threadIdx.x / TPR; rl < kDxPassRows; rl += RPI) {
      const int c = (rl / kWaveRows) * WM + pass * kWaveRows + rl % kWaveRows;
      if (c < vrows && h < a.H) {
        const float* src = (const float*)(smem + rl * kDxRowBytes) + ch * OV;
        const float fs = a.fscale[c0 + c];
        float f[OV];
#pragma unroll
        for (int e = 0; e < OV; e += 4) {
          const f32x4 v = *(const f32x4*)(src + e);
          f[e] = v[0] * fs;
          f[e + 1] = v[1] * fs;
          f[e + 2] = v[2] * fs;
          f[e + 3] = v[3] * fs;
        }
        T* dst = (T*)a.out + a.gmap(a.row0 + c0 + c) + h;
        if (a.accumulate) {
          float o[OV];
          unpack(*(const u32x4*)dst, o, (T*)nullptr);
#pragma unroll
          for (int e = 0; e < OV; ++e) f[e] += o[e];
        }
        *(u32x4*)dst = pack(f, (T*)nullptr);
      }
    }
    __syncthreads();
  }
}

// PART: the tile leaves as fp32 partials (split-K, or the recompute mode's running sum) instead of
// through the row-staged epilogue; one output path per instantiation keeps the register pressure of
// the other out of each kernel.
template <typename T, bool PART>
__global__ __launch_bounds__(NTHR) void k_dx(DxArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kStages * kStageBytes];

  const int mt = (a.rows + TILE - 1) / TILE, nt = (int)((a.H + TILE - 1) / TILE);
  const int t = xcd_remap(blockIdx.x, gridDim.x), per = mt * nt;
  const int split = t / per;
  int tm, tn;
  grouped(t - split * per, mt, nt, kGroupDx, tm, tn);
  const int c0 = tm * TILE, h0 = tn * TILE;

  constexpr int BK = OpK<T>::BK;
  const int nk = (int)(a.V_pad / BK);
  const int kb = split * a.ksteps_per_split;
  const int ke = min(nk, kb + a.ksteps_per_split);
  OpKB<T> la;  // q rows of the chunk (blocked layout), K = v (only this split's K range is loaded)
  la.init((const T*)a.ws + (int64_t)(c0 / TILE) * nk * TILE * BK, ke * BK);
  OpMN<T> lb;  // W: source rows are v (K), columns h
  lb.init((const T*)a.W + h0, a.H, (int)min<int64_t>(a.V, (int64_t)ke * BK), (int)min<int64_t>(TILE, a.H - h0));
  facc acc[TBM][TBN];
  gemm_core<T, kSchedDx>(la, lb, kb, ke, smem, acc);

  // output tile (c0, h0); rows past the chunk and columns past H are dropped
  const int vrows = min(TILE, a.rows - c0), ncols = (int)min<int64_t>(TILE, a.H - h0);
  if constexpr (!PART) {
    dx_store_tile<T>(a, acc, c0, h0, vrows, smem);
  } else {
    const rsrc_t ro = make_rsrc(a.part + ((int64_t)split * a.rows + c0) * a.H + h0, ((int64_t)vrows * a.H - h0) * 4);
    const AccAddr<4> ad((int)a.H, ncols);
    if (a.part_acc) {
      // running fp32 sum over the vocabulary slices of the recompute mode (one split)
#pragma unroll
      for (int i = 0; i < TBM; ++i) {
        float old[TBN][NR];
#pragma unroll
        for (int j = 0; j < TBN; ++j)
#pragma unroll
          for (int r = 0; r < NR; ++r) old[j][r] = bload_f32(ro, ad.col[j], ad.row(i, r));
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int j = 0; j < TBN; ++j) bstore_f32(ro, ad.col[j], ad.row(i, r), acc[i][j][r] + old[j][r]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < TBM; ++i) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int j = 0; j < TBN; ++j) bstore_f32(ro, ad.col[j], ad.row(i, r), acc[i][j][r]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// Fixed-order sum of the split-K partials of grad_hidden times the row's factor f, placed by the row
// map (and added to what the row holds with `accumulate`). Four consecutive columns per thread:
// 16-byte partial loads and one 4-element store (row starts are multiples of 16 bytes, H of 8).
template <typename T>
__global__ __launch_bounds__(256) void k_dx_reduce(const float* part, int splits, int rows, int64_t H, T* out,
                                                    RowMap gmap, int64_t row0, int accumulate, const float* fscale) {
  const int64_t hq = H / 4, g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)rows * hq) return;
  const int c = (int)(g / hq);
  const int64_t h = (g - c * hq) * 4, n = (int64_t)rows * H, i = (int64_t)c * H + h;
  f32x4 s = *(const f32x4*)(part + i);
  for (int k = 1; k < splits; ++k) s += *(const f32x4*)(part + (int64_t)k * n + i);
  s *= fscale[c];
  T* dst = out + gmap(row0 + c) + h;
  if constexpr (sizeof(T) == 2) {
    if (accumulate) {
      const bf16x4 o = *(const bf16x4*)dst;
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += (float)o[e];
    }
    *(u32x2*)dst = pack4_bf16(s[0], s[1], s[2], s[3]);
  } else {
    if (accumulate) s += *(const f32x4*)dst;
    *(f32x4*)dst = s;
  }
}

// ---- grad_W (+)= q^T . hidden_f ---------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NTHR) void k_dw(DwArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kStages * kStageBytes];

  const int mt = (int)((a.V + TILE - 1) / TILE), nt = (int)((a.H + TILE - 1) / TILE);
  const int nk = (a.rows + OpMN<T>::BK - 1) / OpMN<T>::BK;
  int tm, tn, kb = 0, ke = nk, part = -1, ti = 0;
  if ((int)blockIdx.x < a.full) {
    grouped(xcd_remap(blockIdx.x, a.full), mt, nt, kGroupDw, tm, tn);
  } else {
    // a part of one of the last wave's tiles: K steps [nk p / S, nk (p + 1) / S)
    const int e = (int)blockIdx.x - a.full;
    ti = e / a.tail_splits;
    part = e % a.tail_splits;
    grouped(a.full + ti, mt, nt, kGroupDw, tm, tn);
    kb = (int)((int64_t)nk * part / a.tail_splits);
    ke = (int)((int64_t)nk * (part + 1) / a.tail_splits);
  }
  const int v0 = tm * TILE, h0 = tn * TILE;

  // only the block's K range is loaded: the rounded-up steps past ke of the unrolled loop load zeros
  const int kend = min(a.rows, ke * OpMN<T>::BK);
  OpMNB<T> la;  // q^T from the blocked layout: K = chunk rows, M = v; v0 + 256 <= V_pad
  la.init((const T*)a.ws, a.V_pad / kQB<T>, v0, kend);
  OpMN<T> lb;  // hidden_f: source rows are chunk rows (K), columns h
  lb.init((const T*)a.X + h0, a.H, kend, (int)min<int64_t>(TILE, a.H - h0));

  facc acc[TBM][TBN];
  gemm_core<T, kSchedDw>(la, lb, kb, ke, smem, acc);
  if (part >= 0) {
    // a partial tile: the whole 256 x 256 fp32 block (zeros past V or H) to its own slot
    float* pt = a.tail_part + ((int64_t)ti * a.tail_splits + part) * (TILE * TILE);
    const rsrc_t rp = make_rsrc(pt, (int64_t)TILE * TILE * 4);
    const AccAddr<4> ap(TILE, TILE);
#pragma unroll
    for (int i = 0; i < TBM; ++i) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int j = 0; j < TBN; ++j) bstore_f32(rp, ap.col[j], ap.row(i, r), acc[i][j][r]);
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }

  // row-major [V][H] fp32 tile at (v0, h0): written (first chunk) or read-modify-written (later
  // chunks); a row block's loads are all issued before its adds and stores
  const int vrows = (int)min<int64_t>(TILE, a.V - v0), ncols = (int)min<int64_t>(TILE, a.H - h0);
  const rsrc_t rd = make_rsrc(a.dW + (int64_t)v0 * a.H + h0, ((int64_t)vrows * a.H - h0) * 4);
  const AccAddr<4> ad((int)a.H, ncols);
  if (a.accumulate) {
    // software pipeline over the TBM x TBN blocks b = (i, j): the loads of block b + kAhead are
    // issued before block b is added and stored, so kAhead blocks (32 values per lane) of loads cover
    // the memory latency
    constexpr int kAhead = 32 / NR, kNB = TBM * TBN;
    float old[kAhead + 1][NR];
#pragma unroll
    for (int b = 0; b < kAhead; ++b)
#pragma unroll
      for (int r = 0; r < NR; ++r) old[b][r] = bload_f32(rd, ad.col[b % TBN], ad.row(b / TBN, r));
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      if (b + kAhead < kNB) {
        const int bn = b + kAhead;
#pragma unroll
        for (int r = 0; r < NR; ++r) old[bn % (kAhead + 1)][r] = bload_f32(rd, ad.col[bn % TBN], ad.row(bn / TBN, r));
      }
      const int i = b / TBN, j = b % TBN;
#pragma unroll
      for (int r = 0; r < NR; ++r)
        bstore_f32(rd, ad.col[j], ad.row(i, r), acc[i][j][r] + old[b % (kAhead + 1)][r]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < TBM; ++i) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int j = 0; j < TBN; ++j) bstore_f32(rd, ad.col[j], ad.row(i, r), acc[i][j][r]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// grad_W tiles of a split last wave: the partial sums added in a fixed order (part 0, 1, ...), then
// written or added to grad_W. One thread per four consecutive columns of one row of one tile.
__global__ __launch_bounds__(256) void k_dw_tail(const float* part, int splits, int full, int mt, int nt,
                                                 float* dW, int64_t H, int64_t V, int accumulate) {
  constexpr int kQuads = TILE * TILE / 4;  // per tile
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int ti = (int)(g / kQuads), e = (int)(g % kQuads) * 4;
  int tm, tn;
  grouped(full + ti, mt, nt, kGroupDw, tm, tn);
  const int64_t v = (int64_t)tm * TILE + e / TILE, h = (int64_t)tn * TILE + e % TILE;
  if (v >= V || h >= H) return;
  const float* pt = part + (int64_t)ti * splits * (TILE * TILE) + e;
  f32x4 s = *(const f32x4*)pt;
  for (int k = 1; k < splits; ++k) s += *(const f32x4*)(pt + (int64_t)k * (TILE * TILE));
  float* d = dW + v * H + h;
  if ((H & 3) == 0) {  // four whole, 16-byte aligned elements of the row (h and H multiples of 4)
    if (accumulate) s += *(const f32x4*)d;
    *(f32x4*)d = s;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (h + c < H) d[c] = accumulate ? d[c] + s[c] : s[c];
  }
}

// ---- hidden chunk transpose: [rows][H] -> [H][ldt] through a 64 x 64 LDS tile ------------------
// Row r of the chunk is call row row0 + r, found in hidden by the row map. Global memory is read and
// written in 16-byte pieces (H is a multiple of 8 and the row strides of hidden and of the transposed
// chunk are multiples of 16 bytes). A piece of the output that starts before `rows` is written whole:
// its elements past `rows` are zeros, inside the chunk's capacity (a multiple of 256 rows). In LDS a
// tile row takes 4 bytes more than its 64 elements, so that the column reads of a wave fall in
// distinct banks.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* X, RowMap hmap, int64_t row0, int rows, int H, T* XT,
                                                   int64_t ldt) {
  constexpr int KV = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int PR = 64 / KV;              // pieces per 64 elements
  constexpr int ROWB = 64 * (int)sizeof(T) + 4;  // LDS bytes per tile row
  __shared__ __attribute__((aligned(16))) char tile[64 * ROWB];
  __shared__ int64_t roff[64];
  const int r0 = blockIdx.y * 64, h0 = blockIdx.x * 64;
  if (threadIdx.x < 64) roff[threadIdx.x] = r0 + (int)threadIdx.x < rows ? hmap(row0 + r0 + threadIdx.x) : 0;
  __syncthreads();
  u32x4 v[64 * PR / 256];
#pragma unroll
  for (int q = 0; q < 64 * PR / 256; ++q) {
    const int idx = (int)threadIdx.x + 256 * q, r = idx / PR, h = h0 + (idx % PR) * KV;
    v[q] = r0 + r < rows && h < H ? *(const u32x4*)(X + roff[r] + h) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int q = 0; q < 64 * PR / 256; ++q) {
    const int idx = (int)threadIdx.x + 256 * q, r = idx / PR, c = idx % PR;
#pragma unroll
    for (int e = 0; e < 4; ++e) *(u32*)(tile + r * ROWB + c * 16 + 4 * e) = v[q][e];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 64 * PR / 256; ++q) {
    const int idx = (int)threadIdx.x + 256 * q, hh = idx / PR, rc = idx % PR;
    const int h = h0 + hh, r = r0 + rc * KV;
    u32x4 o;
    if constexpr (sizeof(T) == 2) {
      unsigned short e16[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) e16[e] = *(const unsigned short*)(tile + (rc * 8 + e) * ROWB + hh * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (u32)e16[2 * e] | ((u32)e16[2 * e + 1] << 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = *(const u32*)(tile + (rc * 4 + e) * ROWB + hh * 4);
    }
    if (h < H && r < rows) *(u32x4*)(XT + (int64_t)h * ldt + r) = o;
  }
}

// ---- small kernels ----------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Label pre-pass: one block. y32 = label or -1 (ignored or out of range), N, 1/N, status.
__global__ __launch_bounds__(1024) void k_prepass(const int64_t* labels, RowMap lmap, int64_t BT, int64_t V,
                                                  int64_t ignore_index, int reduction, float grad_scale,
                                                  int* y32, DevParams* prm, int* status_out) {
  __shared__ int s_cnt[1024];
  __shared__ int s_bad[1024];
  // thread i takes rows i, i + 1024, ...; the labels of eight of them are loaded together
  constexpr int kB = 8;
  int cnt = 0, bad = 0;
  for (int64_t t0 = threadIdx.x; t0 < BT; t0 += 1024 * kB) {
    int64_t yv[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) yv[k] = t0 + 1024 * k < BT ? labels[lmap(t0 + 1024 * k)] : ignore_index;
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int64_t t = t0 + 1024 * k, y = yv[k];
      const bool counted = y != ignore_index;
      const bool out = counted && (y < 0 || y >= V);
      const bool ok = counted && !out;
      if (t < BT) y32[t] = ok ? (int)y : -1;
      cnt += ok;
      bad |= out;
    }
  }
  s_cnt[threadIdx.x] = cnt;
  s_bad[threadIdx.x] = bad;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      s_cnt[threadIdx.x] += s_cnt[threadIdx.x + o];
      s_bad[threadIdx.x] |= s_bad[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = s_cnt[0];
    prm->n_valid = n;
    prm->ginv = grad_scale * (reduction == 1 ? (n > 0 ? 1.0f / (float)n : 0.0f) : 1.0f);
    prm->status = s_bad[0];
    *status_out = s_bad[0];
  }
}

// Per-row log-sum-exp from the per-(row, 128-wide segment) statistics of the logits epilogue, in a
// fixed order (max over the segments, then the rescaled sum), and the row's loss term (0 on rows that
// do not count). One wave per row: lane l takes segments l, l + 64, ... in that order, loaded eight
// at a time; every lane returns the row's lse and, through max_out, its largest segment reference.
__device__ __forceinline__ float row_lse(const float* m, const float* sp, int nseg, int c, const int* y32,
                                         const float* s_label, float* loss_row, float* lse_out,
                                         float* max_out = nullptr) {
  constexpr int kB = 8;
  const int lane = threadIdx.x & 63;
  float M = kNegInf;
  for (int j0 = lane; j0 < nseg; j0 += 64 * kB) {
    float v[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) v[k] = j0 + 64 * k < nseg ? m[j0 + 64 * k] : kNegInf;
#pragma unroll
    for (int k = 0; k < kB; ++k) M = fmaxf(M, v[k]);
  }
  M = wave_max(M);
  float S = 0.0f;
  for (int j0 = lane; j0 < nseg; j0 += 64 * kB) {
    float mv[kB], sv[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const bool in = j0 + 64 * k < nseg;
      mv[k] = in ? m[j0 + 64 * k] : kNegInf;
      sv[k] = in ? sp[j0 + 64 * k] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kB; ++k)
      if (j0 + 64 * k < nseg) S += sv[k] * ex2((mv[k] - M) * kLog2e);
  }
  S = wave_sum(S);
  const float lse = M + __logf(S);
  if (lane == 0) {
    loss_row[c] = y32[c] >= 0 ? lse - s_label[c] : 0.0f;
    if (lse_out) lse_out[c] = lse;
  }
  if (max_out) *max_out = M;
  return lse;
}

// Reference of each row of a chunk (one wave per row): c = the softcapped label logit, the dot product
// of the row of hidden with the label's row of W in fp32; -inf for rows that do not count (their
// segments then take the segment maximum less kRefSpan as reference, so that their statistics still
// give the row's lse, and their q, at most exp(kRefSpan), meets a zero factor f in the backward).
template <typename T>
__global__ __launch_bounds__(256) void k_rowref(const T* X, RowMap hmap, int64_t row0, int rows, int H, const T* W,
                                                const int* y32, float softcap, float* cref) {
  constexpr int KV = Traits<T>::KV;
  const int lane = threadIdx.x & 63, r = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (r >= rows) return;
  const int y = y32[r];
  if (y < 0) {
    if (lane == 0) cref[r] = kNegInf;
    return;
  }
  const T* x = X + hmap(row0 + r);
  const T* w = W + (int64_t)y * H;
  float acc = 0.0f;
  for (int h = lane * KV; h < H; h += 64 * KV) {
    float a[KV], b[KV];
    unpack(*(const u32x4*)(x + h), a, (T*)nullptr);
    unpack(*(const u32x4*)(w + h), b, (T*)nullptr);
#pragma unroll
    for (int e = 0; e < KV; ++e) acc = fmaf(a[e], b[e], acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) cref[r] = softcap > 0.0f ? softcap * tanh_via_exp(acc / softcap) : acc;
}

// Per row of a chunk (one block per row): lse from the segment statistics and the loss term. Segment j
// holds the pair (r_j, sum of exp(s - r_j)), r_j its reference. A counted row with a reference M =
// max_j r_j above its own c (a segment maximum more than kRefSpan above the label logit) gets M as its
// reference; with `q` (the fused call, where q exists already) its stored q is rescaled to match:
// segment j was stored as exp(s - r_j), so it is multiplied by exp(r_j - M) <= 1. Other rows stop
// after the statistics.
template <typename T>
__global__ __launch_bounds__(256) void k_lse(const float* seg_m, const float* seg_s, int nseg, const int* y32,
                                             const float* s_label, float* loss_row, float* lse, float* cref,
                                             void* q, int64_t qvpad, int rows) {
  using S = typename Traits<T>::S;
  constexpr int KV = Traits<T>::KV;
  const int c = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (c >= rows) return;
  const float* m = seg_m + (int64_t)c * nseg;
  float M;
  row_lse(m, seg_s + (int64_t)c * nseg, nseg, c, y32, s_label, loss_row, lse, &M);
  // every lane has read the old reference (one load instruction of the wave) before lane 0 replaces it
  const float c_old = cref[c];
  if (!(y32[c] >= 0 && M > c_old)) return;  // the same decision in every lane of the wave
  if (lane == 0) cref[c] = M;
  if (!q) return;
  const int64_t nkv = qvpad / kQB<S>;
  for (int k = lane; k < (int)(qvpad / KV); k += 64) {
    const float mj = m[k * KV / kSeg];
    if (mj == kNegInf) continue;  // a segment wholly past V: its q is 0
    const float f = ex2((mj - M) * kLog2e);
    S* p = (S*)q + q_index<S>(c, (int64_t)k * KV, nkv);  // KV consecutive v, inside one block
    float v[KV];
    unpack(*(const u32x4*)p, v, (S*)nullptr);
#pragma unroll
    for (int e = 0; e < KV; ++e) v[e] *= f;
    *(u32x4*)p = pack(v, (S*)nullptr);
  }
}

// Per row of a chunk (one wave per row), after the last q of the row is formed.
//   SCALE: f = g exp(c - lse) (0 for rows that do not count), so that dZ_v = f q_v away from the
//          label; fscale gets f and hidden_f (plain [rows][H]) gets f times the row of hidden.
//   FOLD:  the label's entry of q (when the label lies in the vocabulary columns [v0, v0 + vn) that q
//          holds) becomes dZ_y / f = (softcap derivative) exp(lse - c) expm1(s_y - lse), computed
//          in fp32 from the exact label logit s_y, so that dZ_y = g (p_y - 1) (softcap derivative)
//          keeps its relative precision when p_y is close to 1. Both factors are finite: lse - c is at
//          most ln V + kRefSpan once the reference is within kRefSpan of the row maximum, and
//          expm1(s_y - lse) lies in (-1, 0].
template <typename T>
__global__ __launch_bounds__(256) void k_rowfix(const T* X, RowMap hmap, int64_t row0, int H, T* Xf,
                                                const int* y32, const float* s_label, const float* lse,
                                                const float* cref, const DevParams* prm, float softcap,
                                                float* fscale, void* q, int64_t qvpad, int v0, int vn, int mode,
                                                int rows) {
  using S = typename Traits<T>::S;
  constexpr int KV = Traits<T>::KV;
  const int c = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (c >= rows) return;
  const int y = y32[c];
  const float l = lse[c], cr = cref[c];
  if (mode & 1) {
    const float g = y >= 0 ? prm->ginv : 0.0f;
    const float f = g == 0.0f ? 0.0f : g * ex2((cr - l) * kLog2e);
    if (lane == 0) fscale[c] = f;
    const T* x = X + hmap(row0 + c);
    T* xf = Xf + (int64_t)c * H;
#pragma unroll 4
    for (int h = lane * KV; h < H; h += 64 * KV) {
      float v[KV];
      unpack(*(const u32x4*)(x + h), v, (T*)nullptr);
#pragma unroll
      for (int e = 0; e < KV; ++e) v[e] *= f;
      *(u32x4*)(xf + h) = pack(v, (T*)nullptr);
    }
  }
  if ((mode & 2) && lane == 0 && y >= v0 && y < v0 + vn) {
    const float sy = s_label[c];
    const float t = softcap > 0.0f ? sy / softcap : 0.0f;
    const float val = (1.0f - t * t) * ex2((l - cr) * kLog2e) * expm1f(sy - l);
    ((S*)q)[q_index<S>(c, y - v0, qvpad / kQB<S>)] = (S)val;
  }
}

// Forward-only path: per-row lse and loss term of one chunk (rows row0 .. of the call; one wave per
// row), optionally copied to caller buffers indexed by the call's row.
__global__ __launch_bounds__(256) void k_rows(const float* seg_m, const float* seg_s, int nseg,
                                              const int* y32, const float* s_label, float* loss_row,
                                              float* loss_out, float* lse_out, int rows) {
  const int c = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (c >= rows) return;
  const float lse = row_lse(seg_m + (int64_t)c * nseg, seg_s + (int64_t)c * nseg, nseg, c, y32, s_label,
                            loss_row, lse_out);
  if ((threadIdx.x & 63) == 0 && loss_out) loss_out[c] = y32[c] >= 0 ? lse - s_label[c] : 0.0f;
}

// Fixed-order loss reduction (one block).
__global__ __launch_bounds__(1024) void k_finalize(const float* loss_row, int64_t BT,
                                                   const DevParams* prm, int reduction, float* loss) {
  __shared__ float sh[1024];
  // thread i adds rows i, i + 1024, ... in that order; eight of them are loaded together
  constexpr int kB = 8;
  float s = 0.0f;
  int64_t t = threadIdx.x;
  for (; t + 1024 * (kB - 1) < BT; t += 1024 * kB) {
    float v[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) v[k] = loss_row[t + 1024 * k];
#pragma unroll
    for (int k = 0; k < kB; ++k) s += v[k];
  }
  for (; t < BT; t += 1024) s += loss_row[t];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = prm->n_valid;
    *loss = reduction == 1 ? (n > 0 ? sh[0] / (float)n : 0.0f) : sh[0];
  }
}

__global__ __launch_bounds__(256) void k_zero(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Rows b * sb + off (b < B) of H elements set to zero. Blocks: x over H, y over b (grid-stride).
template <typename T>
__global__ __launch_bounds__(256) void k_zero_rows(T* p, int64_t B, int64_t sb, int64_t off, int64_t H) {
  const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (h >= H) return;
  for (int64_t b = blockIdx.y; b < B; b += gridDim.y) p[b * sb + off + h] = (T)0.0f;
}

}  // namespace

// ---- static scratch of the allocation-free entry point ---------------------------------------
// A file-scope device array: every device the code object is loaded on holds its own copy at its
// own address. Host code never passes the array's name to a kernel or a runtime call (in host code
// it names a host-side stand-in); it uses the address the runtime reports for the current device.
static __device__ __align__(256) char scratch[kScratchBytes];

hipError_t scratch_for_device(int device, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (!out || device < 0 || device >= kMaxDevices) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *out = addr[device];
  return hipSuccess;
}

// ---- launchers ------------------------------------------------------------------------------
hipError_t launch_prepass(const Problem& p, const int64_t* labels, const Work& w, int* status_out,
                          hipStream_t stream) {
  k_prepass<<<1, 1024, 0, stream>>>(labels, p.lmap, p.BT, p.V, p.ignore_index, p.reduction, p.grad_scale,
                                    w.y32, w.params, status_out);
  return hipGetLastError();
}

hipError_t launch_transpose(const Problem& p, const void* hidden, const Work& w, int64_t row0, int64_t rows,
                            hipStream_t stream) {
  const dim3 grid((unsigned)((p.H + 63) / 64), (unsigned)((rows + 63) / 64));
  if (p.dtype == 0)
    k_transpose<__bf16><<<grid, 256, 0, stream>>>((const __bf16*)hidden, p.hmap, row0, (int)rows, (int)p.H,
                                                  (__bf16*)w.xt, w.chunk_cap);
  else
    k_transpose<float><<<grid, 256, 0, stream>>>((const float*)hidden, p.hmap, row0, (int)rows, (int)p.H,
                                                 (float*)w.xt, w.chunk_cap);
  return hipGetLastError();
}

namespace {
FwdArgs fwd_args(const Problem& p, const void* W, const Work& w, int64_t row0, int64_t rows, VSlice vs) {
  if (vs.vn < 0) vs = VSlice{0, p.V};
  const int64_t V_pad = (vs.vn + TILE - 1) / TILE * TILE;
  const size_t esz = p.dtype == 0 ? 2 : 4;
  FwdArgs a;
  a.XT = w.xt;
  a.ldt = w.chunk_cap;
  a.W = (const char*)W + vs.v0 * p.H * (int64_t)esz;
  a.ws = w.ws_e;
  a.seg_m = w.seg_m;
  a.seg_s = w.seg_s;
  a.y = w.y32 + row0;
  a.s_label = w.s_label + row0;
  a.cref = w.cref + row0;
  a.H = p.H;
  a.V = vs.vn;
  a.V_pad = V_pad;
  a.nseg = (int)(V_pad / kSeg);
  a.rows = (int)rows;
  a.yoff = (int)vs.v0;
  a.softcap = p.softcap;
  return a;
}
}  // namespace

hipError_t launch_fwd(const Problem& p, const void* W, const Work& w, int64_t row0, int64_t rows,
                      bool store_q, hipStream_t stream, VSlice vs, bool qonly) {
  const FwdArgs a = fwd_args(p, W, w, row0, rows, vs);
  const unsigned grid = (unsigned)((a.V_pad / TILE) * ((rows + TILE - 1) / TILE));
  if (!store_q && qonly) return hipErrorInvalidValue;
  if (p.dtype == 0) {
    if (!store_q)
      k_fwd<__bf16, false, false><<<grid, NTHR, 0, stream>>>(a);
    else if (qonly)
      k_fwd<__bf16, true, true><<<grid, NTHR, 0, stream>>>(a);
    else
      k_fwd<__bf16, true, false><<<grid, NTHR, 0, stream>>>(a);
  } else {
    if (!store_q)
      k_fwd<float, false, false><<<grid, NTHR, 0, stream>>>(a);
    else if (qonly)
      k_fwd<float, true, true><<<grid, NTHR, 0, stream>>>(a);
    else
      k_fwd<float, true, false><<<grid, NTHR, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_rowref(const Problem& p, const void* hidden, const void* W, const Work& w, int64_t row0,
                         int64_t rows, hipStream_t stream) {
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (p.dtype == 0)
    k_rowref<__bf16><<<grid, 256, 0, stream>>>((const __bf16*)hidden, p.hmap, row0, (int)rows, (int)p.H,
                                               (const __bf16*)W, w.y32 + row0, p.softcap, w.cref + row0);
  else
    k_rowref<float><<<grid, 256, 0, stream>>>((const float*)hidden, p.hmap, row0, (int)rows, (int)p.H,
                                              (const float*)W, w.y32 + row0, p.softcap, w.cref + row0);
  return hipGetLastError();
}

hipError_t launch_lse(const Problem& p, const Work& w, int64_t row0, int64_t rows, bool rescale_q,
                      hipStream_t stream) {
  void* q = rescale_q ? w.ws_e : nullptr;
  if (p.dtype == 0)
    k_lse<__bf16><<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(w.seg_m, w.seg_s, (int)p.nseg, w.y32 + row0,
                                                                  w.s_label + row0, w.loss_row + row0, w.lse + row0,
                                                                  w.cref + row0, q, p.V_pad, (int)rows);
  else
    k_lse<float><<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(w.seg_m, w.seg_s, (int)p.nseg, w.y32 + row0,
                                                                 w.s_label + row0, w.loss_row + row0, w.lse + row0,
                                                                 w.cref + row0, q, p.V_pad, (int)rows);
  return hipGetLastError();
}

hipError_t launch_rowfix(const Problem& p, const void* hidden, const Work& w, int64_t row0, int64_t rows,
                         hipStream_t stream, VSlice vs, int mode) {
  if (vs.vn < 0) vs = VSlice{0, p.V};
  const int64_t qvpad = (vs.vn + TILE - 1) / TILE * TILE;
  if (p.dtype == 0)
    k_rowfix<__bf16><<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(
        (const __bf16*)hidden, p.hmap, row0, (int)p.H, (__bf16*)w.xf, w.y32 + row0, w.s_label + row0, w.lse + row0,
        w.cref + row0, w.params, p.softcap, w.fscale + row0, w.ws_e, qvpad, (int)vs.v0, (int)vs.vn, mode, (int)rows);
  else
    k_rowfix<float><<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(
        (const float*)hidden, p.hmap, row0, (int)p.H, (float*)w.xf, w.y32 + row0, w.s_label + row0, w.lse + row0,
        w.cref + row0, w.params, p.softcap, w.fscale + row0, w.ws_e, qvpad, (int)vs.v0, (int)vs.vn, mode, (int)rows);
  return hipGetLastError();
}

hipError_t launch_rows(const Problem& p, const Work& w, int64_t row0, int64_t rows, float* loss_rows,
                       float* lse_rows, hipStream_t stream) {
  k_rows<<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(w.seg_m, w.seg_s, (int)p.nseg, w.y32 + row0,
                                                         w.s_label + row0, w.loss_row + row0,
                                                         loss_rows ? loss_rows + row0 : nullptr,
                                                         lse_rows ? lse_rows + row0 : nullptr, (int)rows);
  return hipGetLastError();
}

hipError_t launch_dx(const Problem& p, const void* W, const Work& w, void* grad_hidden, int64_t row0,
                     int64_t rows, int splits, hipStream_t stream, VSlice vs, int part_mode) {
  if (vs.vn < 0) vs = VSlice{0, p.V};
  const int64_t V_pad = (vs.vn + TILE - 1) / TILE * TILE;
  const size_t esz = p.dtype == 0 ? 2 : 4;
  const int nk = (int)(V_pad * (int64_t)esz / kStepBytes);
  if (part_mode != 0 && splits != 1) return hipErrorInvalidValue;
  DxArgs a;
  a.W = (const char*)W + vs.v0 * p.H * (int64_t)esz;
  a.ws = w.ws_e;
  a.fscale = w.fscale + row0;
  a.out = grad_hidden;
  a.gmap = p.gmap;
  a.row0 = row0;
  a.accumulate = p.acc_gh ? 1 : 0;
  a.part = w.dx_part;
  a.H = p.H;
  a.V = vs.vn;
  a.V_pad = V_pad;
  a.rows = (int)rows;
  a.splits = splits;
  a.ksteps_per_split = (nk + splits - 1) / splits;
  a.part_out = part_mode != 0 ? 1 : 0;
  a.part_acc = part_mode == 2 ? 1 : 0;
  const unsigned tiles = (unsigned)(((rows + TILE - 1) / TILE) * ((p.H + TILE - 1) / TILE));
  const bool part = a.splits != 1 || a.part_out;
  if (p.dtype == 0) {
    if (part)
      k_dx<__bf16, true><<<tiles * splits, NTHR, 0, stream>>>(a);
    else
      k_dx<__bf16, false><<<tiles * splits, NTHR, 0, stream>>>(a);
  } else {
    if (part)
      k_dx<float, true><<<tiles * splits, NTHR, 0, stream>>>(a);
    else
      k_dx<float, false><<<tiles * splits, NTHR, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_dx_reduce(const Problem& p, const Work& w, void* grad_hidden, int64_t row0, int64_t rows,
                            int splits, hipStream_t stream) {
  const int acc = p.acc_gh ? 1 : 0;
  // every output row starts on a multiple of 16 bytes (the entry points check the strides)
  const RowMap& m = p.gmap;
  if ((p.H & 3) != 0 || (m.sb & 3) != 0 || (m.st & 3) != 0 || (m.base & 3) != 0 || (((uintptr_t)grad_hidden) & 15) != 0)
    return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((rows * (p.H / 4) + 255) / 256);
  if (p.dtype == 0)
    k_dx_reduce<__bf16><<<grid, 256, 0, stream>>>(w.dx_part, splits, (int)rows, p.H, (__bf16*)grad_hidden, p.gmap,
                                                  row0, acc, w.fscale + row0);
  else
    k_dx_reduce<float><<<grid, 256, 0, stream>>>(w.dx_part, splits, (int)rows, p.H, (float*)grad_hidden, p.gmap,
                                                 row0, acc, w.fscale + row0);
  return hipGetLastError();
}

hipError_t launch_zero_rows(const Problem& p, void* grad_hidden, int64_t B, int64_t off, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  const dim3 grid((unsigned)((p.H + 255) / 256), (unsigned)(B < 65535 ? B : 65535));
  if (p.dtype == 0)
    k_zero_rows<__bf16><<<grid, 256, 0, stream>>>((__bf16*)grad_hidden, B, p.gmap.sb, off, p.H);
  else
    k_zero_rows<float><<<grid, 256, 0, stream>>>((float*)grad_hidden, B, p.gmap.sb, off, p.H);
  return hipGetLastError();
}

int dw_tail_plan(int64_t V, int64_t H, int64_t rows, int dtype, int ncu, int* tail) {
  // a last wave under half full is split along K, into at most 4 parts of at least 2 ring depths
  const int64_t tiles = ((V + TILE - 1) / TILE) * ((H + TILE - 1) / TILE);
  if (ncu <= 0) ncu = 256;
  const int t = (int)(tiles % ncu);
  const int64_t bk = kStepBytes / (dtype == 0 ? 2 : 4), nk = (rows + bk - 1) / bk;
  int splits = t > 0 && 2 * t <= ncu ? ncu / t : 1;
  if (splits > 4) splits = 4;
  while (splits > 1 && nk / splits < 2 * kStages) --splits;
  *tail = splits > 1 ? t : 0;
  return splits;
}

hipError_t launch_dw(const Problem& p, const Work& w, float* grad_W, int64_t rows, bool accumulate,
                     hipStream_t stream, VSlice vs) {
  if (vs.vn < 0) vs = VSlice{0, p.V};
  const int64_t V_pad = (vs.vn + TILE - 1) / TILE * TILE;
  DwArgs a;
  a.X = w.xf;  // f times the chunk's rows of hidden, [rows][H]
  a.ws = w.ws_e;
  a.dW = grad_W + vs.v0 * p.H;
  a.H = p.H;
  a.V = vs.vn;
  a.V_pad = V_pad;
  a.rows = (int)rows;
  a.accumulate = accumulate ? 1 : 0;
  const int mt = (int)((vs.vn + TILE - 1) / TILE), nt = (int)((p.H + TILE - 1) / TILE), tiles = mt * nt;
  int tail = 0;
  const int splits = w.dw_tail ? dw_tail_plan(vs.vn, p.H, rows, p.dtype, p.ncu, &tail) : 1;
  a.full = splits > 1 ? tiles - tail : tiles;
  a.tail_splits = splits;
  a.tail_part = w.dw_tail;
  const unsigned grid = (unsigned)(a.full + (splits > 1 ? tail * splits : 0));
  if (p.dtype == 0)
    k_dw<__bf16><<<grid, NTHR, 0, stream>>>(a);
  else
    k_dw<float><<<grid, NTHR, 0, stream>>>(a);
  if (splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_dw_tail<<<(unsigned)tail * (TILE * TILE / 4 / 256), 256, 0, stream>>>(w.dw_tail, splits, a.full, mt, nt,
                                                                           a.dW, p.H, vs.vn, a.accumulate);
  }
  return hipGetLastError();
}

hipError_t launch_finalize(const Problem& p, const Work& w, float* loss, hipStream_t stream) {
  k_finalize<<<1, 1024, 0, stream>>>(w.loss_row, p.BT, w.params, p.reduction, loss);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* ptr, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  k_zero<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(ptr, n);
  return hipGetLastError();
}

}  // namespace flce
