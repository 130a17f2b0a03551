// HIP kernels (gfx950 / CDNA4) for fused linear + cross-entropy, forward and backward.
//
// The computation follows the PR description of "[AOTAutograd] tweak min-cut partitioner to avoid
// saving softmax output" (PyTorch PR #126348): the linear layer gives the softmax input, per-row
// max and sum statistics are formed from it, only the label's entry is needed for the loss, and
// the backward pass rebuilds the softmax from the softmax input and the small max/sum tensors
// instead of reading a saved softmax output. Here that happens per BT chunk:
//
//   k_fwd     Z^T tile = W_tile . X_tile^T on MFMA (bf16 -> fp32), epilogue: optional softcap,
//             per-(row, 128-wide V segment) max and sum of exp, and one 16-bit store per logit of
//             q = exp(s - segment max) * (softcap derivative). No [BT, V] tensor exists.
//   k_merge   per row: lse from the segment statistics, loss term, and the per-segment scale
//             g * exp(segment max - lse) that turns q into dZ.
//   k_dx      grad_hidden chunk = dZ . W on MFMA; the A-operand loader rebuilds dZ tiles in registers
//             from q, the scale and the label (no dlogits tensor is stored).
//   k_dw      grad_W (+)= dZ^T . X on MFMA; both operands are transposed in registers on the way to
//             LDS, dZ rebuilt the same way; fp32 accumulation in place across chunks.
//
// One GEMM core serves the three products: 256 threads (4 waves of 64) compute a 256 x 256 tile,
// each wave a 128 x 128 quarter as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (or 32x32x2f32 for
// fp32 inputs). Operands are staged through a double-buffered, XOR-swizzled LDS tile of 128 bytes
// of K per row; every operand reaches LDS as 16-byte K-contiguous chunks.
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
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int NTHR = 256;        // threads per GEMM block
constexpr int KCH = 8;           // 16-byte chunks per LDS tile row per k-step (128 bytes of K)
constexpr int TILE = kTile;      // 256
constexpr int WT = TILE / 2;     // wave tile (128)
constexpr int TB = WT / 32;      // 32x32 MFMA blocks per wave tile side (4)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

template <typename T> struct Traits;
template <> struct Traits<__bf16> {
  using S = _Float16;                 // workspace element type
  static constexpr int KV = 8;        // elements per 16-byte chunk
};
template <> struct Traits<float> {
  using S = float;
  static constexpr int KV = 4;
};

__device__ __forceinline__ int swz(int row, int kc) {
  // 8 chunks per 128-byte row; XOR with both the low and the next 3 bits of the row so that
  // 16 consecutive rows read at one chunk index, and 8 rows 8 apart written at one chunk index,
  // all land on distinct bank groups.
  return (row << 3) | (kc ^ ((row ^ (row >> 3)) & 7));
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh from its definition through e^{2x}; saturates to +-1 for large |x|.
__device__ __forceinline__ float tanh_via_exp(float x) {
  const float e = ex2(2.0f * kLog2e * x);
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---- MFMA on one 16-byte chunk of K per lane --------------------------------------------------
__device__ __forceinline__ void mma(f32x16& acc, u32x4 a, u32x4 b, __bf16*) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, u32x4 a, u32x4 b, float*) {
  const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
  // lane half h holds k = 4h .. 4h+3 of this 8-wide K slice in both operands; each of the four
  // K=2 MFMAs pairs the e-th element of both halves, so A and B see the same k assignment.
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[e], fb[e], acc, 0, 0, 0);
}

// ---- 16-byte chunk conversions -------------------------------------------------------------
__device__ __forceinline__ void unpack(u32x4 v, float (&f)[8], _Float16*) {
  const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
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

// In-register transpose of a KV x KV block: in[k] holds elements (k, n = 0..KV-1) of a row of the
// source; out[n] receives elements (k = 0..KV-1, n). 2-byte elements: one v_perm_b32 per dword.
__device__ __forceinline__ void transpose(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int n = 0; n < 8; ++n) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32 lo = in[2 * w][n >> 1], hi = in[2 * w + 1][n >> 1];
      out[n][w] = (n & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                          : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
  }
}
__device__ __forceinline__ void transpose(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int k = 0; k < 4; ++k) out[n][k] = in[k][n];
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

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

// ---- operand loaders: global -> registers (load) -> LDS chunks (store) ------------------------
// K-contiguous rows: tile row r is source row r (stride ld), k-step ks covers 8*KV elements.
template <typename T>
struct LoadK {
  static constexpr int KV = 16 / sizeof(T), N = TILE * KCH / NTHR;  // 8 chunks per thread
  const T* p;
  int64_t ld;
  int rows;   // valid tile rows
  int kmax;   // valid K elements
  u32x4 r[N];
  __device__ __forceinline__ void load(int ks) {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int q = it * NTHR + threadIdx.x, row = q >> 3, kc = q & 7;
      const int k = ks * KCH * KV + kc * KV;
      r[it] = (row < rows && k < kmax) ? *(const u32x4*)(p + (int64_t)row * ld + k) : zero4();
    }
  }
  __device__ __forceinline__ void store(u32x4* s) const {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int q = it * NTHR + threadIdx.x;
      s[swz(q >> 3, q & 7)] = r[it];
    }
  }
};

// Source stored with the tile's N index contiguous and K as its row index (MN-contiguous):
// each task loads a KV (k) x KV (n) block with KV 16-byte loads and transposes it in registers.
template <typename T>
struct LoadT {
  static constexpr int KV = 16 / sizeof(T), NG = TILE / KV, TASKS = NG * KCH, N = TASKS / NTHR;
  const T* p;     // element (k = 0, n = 0) of the tile
  int64_t ld;     // source row stride (elements)
  int kvalid;     // valid k rows counted from k = 0
  int nvalid;     // valid n columns in the tile
  u32x4 r[N][KV];
  __device__ __forceinline__ void load(int ks) {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int t = it * NTHR + threadIdx.x, ng = t % NG, kg = t / NG, n = ng * KV;
#pragma unroll
      for (int kk = 0; kk < KV; ++kk) {
        const int k = ks * KCH * KV + kg * KV + kk;
        r[it][kk] = (k < kvalid && n < nvalid) ? *(const u32x4*)(p + (int64_t)k * ld + n) : zero4();
      }
    }
  }
  __device__ __forceinline__ void store(u32x4* s) const {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int t = it * NTHR + threadIdx.x, ng = t % NG, kg = t / NG;
      u32x4 o[KV];
      transpose(r[it], o);
#pragma unroll
      for (int e = 0; e < KV; ++e) s[swz(ng * KV + e, kg)] = o[e];
    }
  }
};

// dZ rows for the grad_hidden product (M = chunk row c, K = v, K-contiguous in the workspace):
// d = q * scale[c][segment(v)] - [v == y_c] * og_c, formed in fp32 and rounded to T.
template <typename T>
struct LoadDzK {
  using S = typename Traits<T>::S;
  static constexpr int KV = Traits<T>::KV, N = TILE * KCH / NTHR;
  const S* p;           // workspace row 0 of the tile
  int64_t ld;           // V_pad
  int rows;             // valid rows
  const float* scale;   // [rows][nseg], tile row 0
  int nseg;
  int yv[N];
  float og[N];
  u32x4 r[N];
  float sc[N];
  __device__ __forceinline__ void init(const int* y, const float* ogp) {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int row = (it * NTHR + threadIdx.x) >> 3;
      yv[it] = row < rows ? y[row] : -1;
      og[it] = row < rows ? ogp[row] : 0.0f;
    }
  }
  __device__ __forceinline__ void load(int ks) {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int q = it * NTHR + threadIdx.x, row = q >> 3, kc = q & 7;
      const int k = ks * KCH * KV + kc * KV;
      const bool ok = row < rows;
      r[it] = ok ? *(const u32x4*)(p + (int64_t)row * ld + k) : zero4();
      sc[it] = ok ? scale[(int64_t)row * nseg + (k / kSeg)] : 0.0f;
    }
  }
  __device__ __forceinline__ void store(u32x4* s, int ks) const {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int q = it * NTHR + threadIdx.x, row = q >> 3, kc = q & 7;
      const int k = ks * KCH * KV + kc * KV;
      float f[KV];
      unpack(r[it], f, (S*)nullptr);
#pragma unroll
      for (int e = 0; e < KV; ++e) f[e] *= sc[it];
      const unsigned rel = (unsigned)(yv[it] - k);
      if (rel < (unsigned)KV) {
#pragma unroll
        for (int e = 0; e < KV; ++e) f[e] -= (rel == (unsigned)e) ? og[it] : 0.0f;
      }
      s[swz(row, kc)] = pack(f, (T*)nullptr);
    }
  }
};

// dZ^T for the grad_W product (M = v, K = chunk row c): the workspace is [c][v], so each task loads
// KV rows c x KV columns v, forms d per element with the row's scale and label, rounds to T and
// transposes in registers so that LDS holds K(c)-contiguous chunks per v.
template <typename T>
struct LoadDzT {
  using S = typename Traits<T>::S;
  static constexpr int KV = Traits<T>::KV, NG = TILE / KV, TASKS = NG * KCH, N = TASKS / NTHR;
  const S* p;           // workspace element (c = 0, v = v0)
  int64_t ld;           // V_pad
  int rows;             // valid chunk rows (K extent)
  const float* scale;   // [rows][nseg] (chunk row 0)
  int nseg;
  int v0;               // first v of the tile
  const int* y;         // chunk row 0
  const float* ogp;
  u32x4 r[N][KV];
  float sc[N][KV];
  int yv[N][KV];
  float og[N][KV];
  __device__ __forceinline__ void load(int ks) {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int t = it * NTHR + threadIdx.x, ng = t % NG, kg = t / NG;
      const int seg = (v0 + ng * KV) / kSeg;
#pragma unroll
      for (int kk = 0; kk < KV; ++kk) {
        const int c = ks * KCH * KV + kg * KV + kk;
        const bool ok = c < rows;
        r[it][kk] = ok ? *(const u32x4*)(p + (int64_t)c * ld + ng * KV) : zero4();
        sc[it][kk] = ok ? scale[(int64_t)c * nseg + seg] : 0.0f;
        yv[it][kk] = ok ? y[c] : -1;
        og[it][kk] = ok ? ogp[c] : 0.0f;
      }
    }
  }
  __device__ __forceinline__ void store(u32x4* s, int) const {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int t = it * NTHR + threadIdx.x, ng = t % NG, kg = t / NG;
      const int vb = v0 + ng * KV;
      u32x4 d[KV];
#pragma unroll
      for (int kk = 0; kk < KV; ++kk) {
        float f[KV];
        unpack(r[it][kk], f, (S*)nullptr);
#pragma unroll
        for (int e = 0; e < KV; ++e) f[e] *= sc[it][kk];
        const unsigned rel = (unsigned)(yv[it][kk] - vb);
        if (rel < (unsigned)KV) {
#pragma unroll
          for (int e = 0; e < KV; ++e) f[e] -= (rel == (unsigned)e) ? og[it][kk] : 0.0f;
        }
        d[kk] = pack(f, (T*)nullptr);
      }
      u32x4 o[KV];
      transpose(d, o);
#pragma unroll
      for (int e = 0; e < KV; ++e) s[swz(ng * KV + e, kg)] = o[e];
    }
  }
};

// Adapters so that plain loaders and the dZ loaders share one call shape.
template <class L> __device__ __forceinline__ void store_chunks(const L& l, u32x4* s, int) { l.store(s); }
template <typename T> __device__ __forceinline__ void store_chunks(const LoadDzK<T>& l, u32x4* s, int ks) { l.store(s, ks); }
template <typename T> __device__ __forceinline__ void store_chunks(const LoadDzT<T>& l, u32x4* s, int ks) { l.store(s, ks); }

// ---- the MFMA tile core --------------------------------------------------------------------
// acc[i][j] is the 32x32 block (wave_m*128 + 32 i, wave_n*128 + 32 j) of the 256 x 256 tile. In the
// 32x32 MFMA result layout, lane l holds column (l % 32) and, in register r, row
// 8 * (r / 4) + 4 * (l / 32) + r % 4 of its block.
template <typename T, class LA, class LB>
__device__ __forceinline__ void gemm_core(LA& la, LB& lb, int kb, int ke, u32x4* sA, u32x4* sB,
                                          f32x16 (&acc)[TB][TB]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (kb >= ke) return;

  la.load(kb);
  lb.load(kb);
  store_chunks(la, sA, kb);
  store_chunks(lb, sB, kb);
  __syncthreads();

  const int arow = wm * WT + (lane & 31), brow = wn * WT + (lane & 31), half = lane >> 5;
  for (int ks = kb; ks < ke; ++ks) {
    const int cur = (ks - kb) & 1;
    const u32x4* a = sA + cur * TILE * KCH;
    const u32x4* b = sB + cur * TILE * KCH;
    const bool more = ks + 1 < ke;
    if (more) {
      la.load(ks + 1);
      lb.load(ks + 1);
    }
#pragma unroll
    for (int s = 0; s < KCH / 2; ++s) {
      const int kc = 2 * s + half;
      u32x4 fa[TB], fb[TB];
#pragma unroll
      for (int i = 0; i < TB; ++i) fa[i] = a[swz(arow + 32 * i, kc)];
#pragma unroll
      for (int j = 0; j < TB; ++j) fb[j] = b[swz(brow + 32 * j, kc)];
#pragma unroll
      for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) mma(acc[i][j], fa[i], fb[j], (T*)nullptr);
    }
    if (more) {
      store_chunks(la, sA + (cur ^ 1) * TILE * KCH, ks + 1);
      store_chunks(lb, sB + (cur ^ 1) * TILE * KCH, ks + 1);
    }
    __syncthreads();
  }
}

// ---- kernel arguments ------------------------------------------------------------------------
struct FwdArgs {
  const void* X;      // hidden, chunk row 0
  const void* W;
  void* ws;
  float* seg_m;
  float* seg_s;
  int64_t H, V, V_pad;
  int nseg, rows;
  float softcap;
};

struct DxArgs {
  const void* W;
  const void* ws;
  const float* scale;
  const int* y;       // chunk row 0
  const float* og;    // chunk row 0
  void* out;          // grad_hidden, chunk row 0 (splits == 1)
  float* part;        // [splits][rows][H] (splits > 1)
  int64_t H, V, V_pad;
  int nseg, rows, splits, ksteps_per_split;
};

struct DwArgs {
  const void* X;      // hidden, chunk row 0
  const void* ws;
  const float* scale;
  const int* y;
  const float* og;
  float* dW;
  int64_t H, V, V_pad;
  int nseg, rows, accumulate;
};

constexpr int kGroupFwd = 16;
constexpr int kGroupDx = 4;
constexpr int kGroupDw = 8;

// ---- forward: logits tile + softcap + segment statistics + q store -------------------------
template <typename T>
__global__ __launch_bounds__(NTHR) void k_fwd(FwdArgs a) {
  using S = typename Traits<T>::S;
  constexpr int KV = Traits<T>::KV;
  __shared__ u32x4 sA[2 * TILE * KCH];
  __shared__ u32x4 sB[2 * TILE * KCH];

  const int mt = (int)(a.V_pad / TILE), nt = (a.rows + TILE - 1) / TILE;
  int tm, tn;
  grouped(xcd_remap(blockIdx.x, gridDim.x), mt, nt, kGroupFwd, tm, tn);
  const int v0 = tm * TILE, c0 = tn * TILE;

  LoadK<T> la{(const T*)a.W + (int64_t)v0 * a.H, a.H, (int)min<int64_t>(TILE, a.V - v0), (int)a.H, {}};
  LoadK<T> lb{(const T*)a.X + (int64_t)c0 * a.H, a.H, min(TILE, a.rows - c0), (int)a.H, {}};
  f32x16 acc[TB][TB];
  const int nk = (int)((a.H + KCH * KV - 1) / (KCH * KV));
  gemm_core<T>(la, lb, 0, nk, sA, sB, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  const int vw = v0 + wm * WT, seg = vw / kSeg, half = lane >> 5;
  const bool full = vw + WT <= a.V;
  const float cap = a.softcap, icap = cap > 0.0f ? 1.0f / cap : 0.0f;
  S* ws = (S*)a.ws;
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int c = c0 + wn * WT + 32 * j + (lane & 31);
    const bool row_ok = c < a.rows;
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = acc[i][j][r];
        if (cap > 0.0f) s = cap * tanh_via_exp(s * icap);
        acc[i][j][r] = s;
        const int v = vw + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (full || v < a.V) mx = fmaxf(mx, s);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float msl = (mx == kNegInf ? 0.0f : mx) * kLog2e;
    float sum = 0.0f;
    S* dst = ws + (int64_t)c * a.V_pad + vw + 4 * half;
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float q[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float s = acc[i][j][4 * g + rr];
          const int v = vw + 32 * i + 8 * g + 4 * half + rr;
          float e = ex2(s * kLog2e - msl);
          if (!full && v >= a.V) e = 0.0f;
          sum += e;
          const float t = s * icap;
          q[rr] = cap > 0.0f ? e * (1.0f - t * t) : e;
        }
        if (row_ok) {
          if constexpr (sizeof(S) == 2) {
            f16x4 h{(S)q[0], (S)q[1], (S)q[2], (S)q[3]};
            *(u32x2*)(dst + 32 * i + 8 * g) = __builtin_bit_cast(u32x2, h);
          } else {
            *(f32x4*)(dst + 32 * i + 8 * g) = f32x4{q[0], q[1], q[2], q[3]};
          }
        }
      }
    sum += __shfl_xor(sum, 32);
    if (lane < 32 && row_ok) {
      a.seg_m[(int64_t)c * a.nseg + seg] = mx;
      a.seg_s[(int64_t)c * a.nseg + seg] = sum;
    }
  }
}

// ---- grad_hidden = dZ . W ---------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NTHR) void k_dx(DxArgs a) {
  using S = typename Traits<T>::S;
  __shared__ u32x4 sA[2 * TILE * KCH];
  __shared__ u32x4 sB[2 * TILE * KCH];

  const int mt = (a.rows + TILE - 1) / TILE, nt = (int)((a.H + TILE - 1) / TILE);
  const int t = xcd_remap(blockIdx.x, gridDim.x), per = mt * nt;
  const int split = t / per;
  int tm, tn;
  grouped(t - split * per, mt, nt, kGroupDx, tm, tn);
  const int c0 = tm * TILE, h0 = tn * TILE;

  LoadDzK<T> la;
  la.p = (const S*)a.ws + (int64_t)c0 * a.V_pad;
  la.ld = a.V_pad;
  la.rows = min(TILE, a.rows - c0);
  la.scale = a.scale + (int64_t)c0 * a.nseg;
  la.nseg = a.nseg;
  la.init(a.y + c0, a.og + c0);
  LoadT<T> lb{(const T*)a.W + h0, a.H, (int)a.V, (int)min<int64_t>(TILE, a.H - h0), {}};

  const int kb = split * a.ksteps_per_split;
  const int nk = (int)(a.V_pad / (KCH * Traits<T>::KV));
  const int ke = min(nk, kb + a.ksteps_per_split);
  f32x16 acc[TB][TB];
  gemm_core<T>(la, lb, kb, ke, sA, sB, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int h = h0 + wn * WT + 32 * j + (lane & 31);
      if (h >= a.H) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = c0 + wm * WT + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (c >= a.rows) continue;
        const float v = acc[i][j][r];
        if (a.splits == 1) {
          ((T*)a.out)[(int64_t)c * a.H + h] = (T)v;
        } else {
          a.part[((int64_t)split * a.rows + c) * a.H + h] = v;
        }
      }
    }
}

// Fixed-order sum of the split-K partials of grad_hidden.
template <typename T>
__global__ __launch_bounds__(256) void k_dx_reduce(const float* part, int splits, int64_t n, T* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int k = 0; k < splits; ++k) s += part[(int64_t)k * n + i];
  out[i] = (T)s;
}

// ---- grad_W (+)= dZ^T . X -----------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NTHR) void k_dw(DwArgs a) {
  using S = typename Traits<T>::S;
  __shared__ u32x4 sA[2 * TILE * KCH];
  __shared__ u32x4 sB[2 * TILE * KCH];

  const int mt = (int)((a.V + TILE - 1) / TILE), nt = (int)((a.H + TILE - 1) / TILE);
  int tm, tn;
  grouped(xcd_remap(blockIdx.x, gridDim.x), mt, nt, kGroupDw, tm, tn);
  const int v0 = tm * TILE, h0 = tn * TILE;

  LoadDzT<T> la;
  la.p = (const S*)a.ws + v0;
  la.ld = a.V_pad;
  la.rows = a.rows;
  la.scale = a.scale;
  la.nseg = a.nseg;
  la.v0 = v0;
  la.y = a.y;
  la.ogp = a.og;
  LoadT<T> lb{(const T*)a.X + h0, a.H, a.rows, (int)min<int64_t>(TILE, a.H - h0), {}};

  const int nk = (a.rows + KCH * Traits<T>::KV - 1) / (KCH * Traits<T>::KV);
  f32x16 acc[TB][TB];
  gemm_core<T>(la, lb, 0, nk, sA, sB, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int h = h0 + wn * WT + 32 * j + (lane & 31);
      if (h >= a.H) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = v0 + wm * WT + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (v >= a.V) continue;
        float* d = a.dW + (int64_t)v * a.H + h;
        const float val = acc[i][j][r];
        *d = a.accumulate ? *d + val : val;
      }
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
__global__ __launch_bounds__(1024) void k_prepass(const int64_t* labels, int64_t BT, int64_t V,
                                                  int64_t ignore_index, int reduction, int* y32,
                                                  DevParams* prm, int* status_out) {
  __shared__ int s_cnt[1024];
  __shared__ int s_bad[1024];
  int cnt = 0, bad = 0;
  for (int64_t t = threadIdx.x; t < BT; t += 1024) {
    const int64_t y = labels[t];
    const bool counted = y != ignore_index;
    const bool out = counted && (y < 0 || y >= V);
    const bool ok = counted && !out;
    y32[t] = ok ? (int)y : -1;
    cnt += ok;
    bad |= out;
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
    prm->ginv = reduction == 1 ? (n > 0 ? 1.0f / (float)n : 0.0f) : 1.0f;
    prm->status = s_bad[0];
    *status_out = s_bad[0];
  }
}

// Label logit per row (one wave per row): s_y = softcap(x . W[y]) and og = g * ds_y/dz_y.
template <typename T>
__global__ __launch_bounds__(256) void k_label_logit(const T* X, const T* W, const int* y32,
                                                     const DevParams* prm, int64_t BT, int64_t H,
                                                     float softcap, float* s_label, float* og) {
  constexpr int KV = 16 / sizeof(T);
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= BT) return;
  const int y = y32[t];
  if (y < 0) {
    if (lane == 0) {
      s_label[t] = 0.0f;
      og[t] = 0.0f;
    }
    return;
  }
  const T* x = X + t * H;
  const T* w = W + (int64_t)y * H;
  float acc = 0.0f;
  for (int64_t h = (int64_t)lane * KV; h < H; h += 64 * KV) {
    float fx[KV], fw[KV];
    const u32x4 vx = *(const u32x4*)(x + h), vw = *(const u32x4*)(w + h);
    if constexpr (sizeof(T) == 2) {
      const bf16x8 bx = __builtin_bit_cast(bf16x8, vx), bw = __builtin_bit_cast(bf16x8, vw);
#pragma unroll
      for (int e = 0; e < KV; ++e) {
        fx[e] = (float)bx[e];
        fw[e] = (float)bw[e];
      }
    } else {
      const f32x4 bx = __builtin_bit_cast(f32x4, vx), bw = __builtin_bit_cast(f32x4, vw);
#pragma unroll
      for (int e = 0; e < KV; ++e) {
        fx[e] = bx[e];
        fw[e] = bw[e];
      }
    }
#pragma unroll
    for (int e = 0; e < KV; ++e) acc = fmaf(fx[e], fw[e], acc);
  }
  const float z = wave_sum(acc);
  if (lane == 0) {
    const float g = prm->ginv;
    if (softcap > 0.0f) {
      const float th = tanh_via_exp(z / softcap);
      s_label[t] = softcap * th;
      og[t] = g * (1.0f - th * th);
    } else {
      s_label[t] = z;
      og[t] = g;
    }
  }
}

// Row merge (one wave per row): lse from the segment statistics, loss term, per-segment scale.
__global__ __launch_bounds__(256) void k_merge(float* seg_m, const float* seg_s, int nseg, int rows,
                                               const int* y32, const float* s_label,
                                               const DevParams* prm, float* loss_row) {
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (c >= rows) return;
  float* m = seg_m + (int64_t)c * nseg;
  const float* s = seg_s + (int64_t)c * nseg;
  float M = kNegInf;
  for (int j = lane; j < nseg; j += 64) M = fmaxf(M, m[j]);
  M = wave_max(M);
  const float Ml = M * kLog2e;
  float S = 0.0f;
  for (int j = lane; j < nseg; j += 64) S += s[j] * ex2(m[j] * kLog2e - Ml);
  S = wave_sum(S);
  const float lse = M + __logf(S);
  const bool valid = y32[c] >= 0;
  const float g = valid ? prm->ginv : 0.0f;
  const float lsel = lse * kLog2e;
  for (int j = lane; j < nseg; j += 64) m[j] = g * ex2(m[j] * kLog2e - lsel);
  if (lane == 0) loss_row[c] = valid ? lse - s_label[c] : 0.0f;
}

// Fixed-order loss reduction (one block).
__global__ __launch_bounds__(1024) void k_finalize(const float* loss_row, int64_t BT,
                                                   const DevParams* prm, int reduction, float* loss) {
  __shared__ float sh[1024];
  float s = 0.0f;
  for (int64_t t = threadIdx.x; t < BT; t += 1024) s += loss_row[t];
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

}  // namespace

// ---- launchers ------------------------------------------------------------------------------
hipError_t launch_prepass(const Problem& p, const int64_t* labels, const Work& w, int* status_out,
                          hipStream_t stream) {
  k_prepass<<<1, 1024, 0, stream>>>(labels, p.BT, p.V, p.ignore_index, p.reduction, w.y32, w.params,
                                    status_out);
  return hipGetLastError();
}

hipError_t launch_label_logit(const Problem& p, const void* hidden, const void* W, const Work& w,
                              hipStream_t stream) {
  const unsigned grid = (unsigned)((p.BT + 3) / 4);
  if (p.dtype == 0)
    k_label_logit<__bf16><<<grid, 256, 0, stream>>>((const __bf16*)hidden, (const __bf16*)W, w.y32,
                                                    w.params, p.BT, p.H, p.softcap, w.s_label, w.og);
  else
    k_label_logit<float><<<grid, 256, 0, stream>>>((const float*)hidden, (const float*)W, w.y32, w.params,
                                                   p.BT, p.H, p.softcap, w.s_label, w.og);
  return hipGetLastError();
}

hipError_t launch_fwd(const Problem& p, const void* hidden, const void* W, const Work& w, int64_t row0,
                      int64_t rows, hipStream_t stream) {
  const size_t esz = p.dtype == 0 ? 2 : 4;
  FwdArgs a;
  a.X = (const char*)hidden + row0 * p.H * esz;
  a.W = W;
  a.ws = w.ws_e;
  a.seg_m = w.seg_m;
  a.seg_s = w.seg_s;
  a.H = p.H;
  a.V = p.V;
  a.V_pad = p.V_pad;
  a.nseg = (int)p.nseg;
  a.rows = (int)rows;
  a.softcap = p.softcap;
  const unsigned grid = (unsigned)((p.V_pad / TILE) * ((rows + TILE - 1) / TILE));
  if (p.dtype == 0)
    k_fwd<__bf16><<<grid, NTHR, 0, stream>>>(a);
  else
    k_fwd<float><<<grid, NTHR, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_merge(const Problem& p, const Work& w, int64_t row0, int64_t rows, hipStream_t stream) {
  const unsigned grid = (unsigned)((rows + 3) / 4);
  k_merge<<<grid, 256, 0, stream>>>(w.seg_m, w.seg_s, (int)p.nseg, (int)rows, w.y32 + row0,
                                    w.s_label + row0, w.params, w.loss_row + row0);
  return hipGetLastError();
}

hipError_t launch_dx(const Problem& p, const void* W, const Work& w, void* grad_hidden, int64_t row0,
                     int64_t rows, int splits, hipStream_t stream) {
  const size_t esz = p.dtype == 0 ? 2 : 4;
  const int kv = p.dtype == 0 ? 8 : 4;
  const int nk = (int)(p.V_pad / (KCH * kv));
  DxArgs a;
  a.W = W;
  a.ws = w.ws_e;
  a.scale = w.seg_m;
  a.y = w.y32 + row0;
  a.og = w.og + row0;
  a.out = (char*)grad_hidden + row0 * p.H * esz;
  a.part = w.dx_part;
  a.H = p.H;
  a.V = p.V;
  a.V_pad = p.V_pad;
  a.nseg = (int)p.nseg;
  a.rows = (int)rows;
  a.splits = splits;
  a.ksteps_per_split = (nk + splits - 1) / splits;
  const unsigned tiles = (unsigned)(((rows + TILE - 1) / TILE) * ((p.H + TILE - 1) / TILE));
  if (p.dtype == 0)
    k_dx<__bf16><<<tiles * splits, NTHR, 0, stream>>>(a);
  else
    k_dx<float><<<tiles * splits, NTHR, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_dx_reduce(const Problem& p, const Work& w, void* grad_hidden, int64_t row0, int64_t rows,
                            int splits, hipStream_t stream) {
  const size_t esz = p.dtype == 0 ? 2 : 4;
  void* out = (char*)grad_hidden + row0 * p.H * esz;
  const int64_t n = rows * p.H;
  const unsigned g2 = (unsigned)((n + 255) / 256);
  if (p.dtype == 0)
    k_dx_reduce<__bf16><<<g2, 256, 0, stream>>>(w.dx_part, splits, n, (__bf16*)out);
  else
    k_dx_reduce<float><<<g2, 256, 0, stream>>>(w.dx_part, splits, n, (float*)out);
  return hipGetLastError();
}

hipError_t launch_dw(const Problem& p, const void* hidden, const Work& w, float* grad_W, int64_t row0,
                     int64_t rows, bool accumulate, hipStream_t stream) {
  const size_t esz = p.dtype == 0 ? 2 : 4;
  DwArgs a;
  a.X = (const char*)hidden + row0 * p.H * esz;
  a.ws = w.ws_e;
  a.scale = w.seg_m;
  a.y = w.y32 + row0;
  a.og = w.og + row0;
  a.dW = grad_W;
  a.H = p.H;
  a.V = p.V;
  a.V_pad = p.V_pad;
  a.nseg = (int)p.nseg;
  a.rows = (int)rows;
  a.accumulate = accumulate ? 1 : 0;
  const unsigned grid = (unsigned)(((p.V + TILE - 1) / TILE) * ((p.H + TILE - 1) / TILE));
  if (p.dtype == 0)
    k_dw<__bf16><<<grid, NTHR, 0, stream>>>(a);
  else
    k_dw<float><<<grid, NTHR, 0, stream>>>(a);
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
