// kernels_proj.hip -- the dense projections around the operator, on the
// matrix cores.
//
// In-projection (paper digest, irregular6612.github.io, section "방법 (Method)",
// framework figure: one projection of width (N+1)D gives v and the gates;
// homemade-llm "02. 3つの Hyena 演算子", section 2: each projected stream is
// featurised by its own short convolution):
//   Z[b][t][c] = sum_k u[b][t][k] W[c][k] + bias[c],
//   S[b][c][t] = sum_{j<T} w[c][j] Z[b][t-j][c]      (Z = 0 before t = 0),
// stored as stream c / D, channel c % D of a [B][D][L] (time-fastest) array.
// Out-projection (same section of homemade-llm, the dense matrix M):
//   out[b][t][e] = sum_d W[e][d] y[b][d][t] + bias[e].
//
// Both compute 128 x 128 output tiles per 256-thread workgroup: four waves of
// 64 x 64, each a 2 x 2 set of 32 x 32 MFMA accumulators (fp32 operands:
// v_mfma_f32_32x32x2f32; bf16 operands: v_mfma_f32_32x32x16_bf16 with fp32
// accumulation).  Operand tiles go global -> registers -> LDS, the next
// k-stage's loads in flight while the current stage's MFMAs run.  The
// in-projection walks a strip of consecutive time tiles and carries the last
// rows of Z from tile to tile, so the short convolution needs no recomputed
// halo except at a strip's first tile.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "fft_engine.hpp"
#include "launch.hpp"

namespace hyena {
namespace {

constexpr int TM = 128, TN = 128, TT = 256;   // tile rows, tile columns, threads
constexpr int HALO = 16;                       // carried Z rows (T - 1 <= 15)
constexpr int ZLD = HALO + TM + 1;             // epilogue row stride (odd: conflict-free column writes)

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int IOT> struct Op;
template <> struct Op<0> {       // fp32: 32 k per stage, rows padded to 33
  using E = float;
  static constexpr int BK = 32, LDK = 33, W = 4;
};
template <> struct Op<1> {       // bf16: 64 k per stage, rows padded to 72 (16-byte aligned)
  using E = uint16_t;
  static constexpr int BK = 64, LDK = 72, W = 8;
};

__device__ __forceinline__ float ld_f(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_f(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }

template <int IOT>
__device__ __forceinline__ void st_f(void* p, int64_t i, float v) {
  if constexpr (IOT == 0) static_cast<float*>(p)[i] = v;
  else static_cast<uint16_t*>(p)[i] = (uint16_t)bf16x2_bits(v, 0.f);
}

// Register stage of a 128-row x BK tile whose rows are contiguous in k: row r
// at src[roff + r*ld + k].  Rows outside [0, rhi) and k >= K read as zero.
// VEC: K is a multiple of the item width W, so an item is all in or all out.
template <int IOT, bool VEC>
struct RowStage {
  using E = typename Op<IOT>::E;
  static constexpr int W = Op<IOT>::W, LDK = Op<IOT>::LDK;
  u32x4 v[4];
  __device__ __forceinline__ void load(const E* src, int64_t roff, int64_t ld, int rhi, int k0, int K, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + TT * i;
      const int r = idx >> 3, k = k0 + (idx & 7) * W;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (r < rhi) {
        const E* p = src + roff + (int64_t)r * ld + k;
        if constexpr (VEC) {
          if (k < K) w = *reinterpret_cast<const u32x4*>(p);
        } else if constexpr (IOT == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (k + e < K) ? __float_as_uint(p[e]) : 0u;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k + e < K) w[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
        }
      }
      v[i] = w;
    }
  }
  __device__ __forceinline__ void store(E* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + TT * i;
      const int r = idx >> 3, q = (idx & 7) * W;
      if constexpr (IOT == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lds[r * LDK + q + e] = __uint_as_float(v[i][e]);
      } else {
        *reinterpret_cast<u32x4*>(lds + r * LDK + q) = v[i];
      }
    }
  }
};

// One k-stage of MFMAs over the LDS tiles into the wave's 2 x 2 accumulators.
// A is row-major [m][k] (stride LDK), or for fp32 with AT k-major [k][m]
// (stride TM + 4); B is row-major [n][k].
template <int IOT, bool AT>
struct Mma;

template <bool AT>
struct Mma<0, AT> {
  static __device__ __forceinline__ void run(f32x16 (&acc)[2][2], const float* As, const float* Bs, int wm, int wn,
                                             int lane) {
#pragma unroll
    for (int kk = 0; kk < Op<0>::BK / 2; ++kk) {
      const int k = 2 * kk + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = wm * 64 + i * 32 + (lane & 31);
        a[i] = AT ? As[k * (TM + 4) + m] : As[m * Op<0>::LDK + k];
        b[i] = Bs[(wn * 64 + i * 32 + (lane & 31)) * Op<0>::LDK + k];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
};

template <>
struct Mma<1, false> {
  static __device__ __forceinline__ void run(f32x16 (&acc)[2][2], const uint16_t* As, const uint16_t* Bs, int wm,
                                             int wn, int lane) {
#pragma unroll
    for (int kk = 0; kk < Op<1>::BK / 16; ++kk) {
      const int k = 16 * kk + 8 * (lane >> 5);
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 32 + (lane & 31)) * Op<1>::LDK + k);
        b[i] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 64 + i * 32 + (lane & 31)) * Op<1>::LDK + k);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
};

// Accumulator element r of lane `lane` in a 32 x 32 block: row 8(r/4) + 4(lane/32) + r%4, column lane%32.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <class E, bool VEC>
__device__ __forceinline__ float dot_row(const E* x, const E* w, int K) {
  float acc = 0.f;
  if constexpr (VEC && sizeof(E) == 4) {
    for (int k = 0; k < K; k += 4) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(x + k), b = *reinterpret_cast<const u32x4*>(w + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(a[e]), __uint_as_float(b[e]), acc);
    }
  } else if constexpr (VEC) {
    for (int k = 0; k < K; k += 8) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(x + k), b = *reinterpret_cast<const u32x4*>(w + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16), acc);
        acc = fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(b[e] & 0xffff0000u), acc);
      }
    }
  } else {
    for (int k = 0; k < K; ++k) acc = fmaf(ld_f(x, k), ld_f(w, k), acc);
  }
  return acc;
}

// Workgroup -> (row job, column block) map.  Workgroup w runs on XCD w mod 8,
// and each XCD has its own L2.  The 8 XCDs form a grid of (8 / cg) row-job
// groups x cg column-block groups; XCD x takes row jobs [(x / cg) * spx, +spx)
// and column blocks [(x % cg) * cbx, +cbx), its workgroups w = x + 8k walking
// them column block fastest.  An operand tile is then read into few L2s
// (A-rows by cg of them, weight blocks by 8 / cg), instead of into most of
// the eight.  Slots past the end of either range are idle.  The map is a
// permutation of the jobs whatever the hardware does with it.
struct XcdTiles {
  int cg, spx, cbx;
  __device__ __forceinline__ bool tile_of(int w, int jobs, int cbs, int& job, int& cb) const {
    const int x = w & 7, k = w >> 3;
    const int jl = k / cbx;
    job = (x / cg) * spx + jl;
    cb = (x % cg) * cbx + (k - jl * cbx);
    return jl < spx && job < jobs && cb < cbs;
  }
};

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// The map for `jobs` row jobs and `cbs` column blocks whose operand tiles
// are the same size: the split of the 8 XCDs that keeps the fewest tiles
// live per L2 (spx + cbx), then the fewest workgroups.
static XcdTiles plan_xcd(int jobs, int cbs, int64_t& grid) {
  XcdTiles best{1, jobs, cbs};
  int64_t best_cost = -1;
  for (int cg = 1; cg <= 8; cg *= 2) {
    const int spx = ceil_div(jobs, 8 / cg), cbx = ceil_div(cbs, cg);
    const int64_t g = 8LL * spx * cbx, cost = (int64_t)(spx + cbx) << 32 | g;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = XcdTiles{cg, spx, cbx};
      grid = g;
    }
  }
  return best;
}

// In-projection epilogue for one half (64 columns) of a tile: Z of column n
// sits at Zs[n*ZLD + HALO + m] (m = 0..127, tile rows) after HALO carried
// rows, and taps[c][j] = w[c][j] (zero for j >= T).  K >= T taps are applied.
template <int IOT, int K>
__device__ __forceinline__ void fir_store(const InProjArgs& a, const float* Zs, const float (*taps)[HALO], int h,
                                          int c0, int b, int64_t t0, int64_t te, int wave, int lane) {
  constexpr int G = K <= 4 ? 4 : 1;                   // columns per step
  const int D = a.D, C = a.C;
  const int64_t L = a.L;
  for (int n0 = wave; n0 < 64; n0 += G * (TT / 64)) {
    float o0[G], o1[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int n = n0 + g * (TT / 64);
      const float* zr = Zs + n * ZLD + HALO + 2 * lane;
      const float* wc = taps[64 * h + n];
      float z[K + 1];                                 // z[k] = Z(t + 1 - k), t = 2 lane
#pragma unroll
      for (int k = 0; k <= K; ++k) z[k] = zr[1 - k];
      o0[g] = 0.f;
      o1[g] = 0.f;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const float wj = wc[j];
        o0[g] = fmaf(wj, z[j + 1], o0[g]);
        o1[g] = fmaf(wj, z[j], o1[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // the column is the wave's own (uniform): the stream pointer is then a
      // scalar load, not a per-lane one that each masked store waits for
      const int c = __builtin_amdgcn_readfirstlane(c0 + 64 * h + n0 + g * (TT / 64));
      if (c >= C) break;
      const int s = c / D, d = c - (c / D) * D;
      void* dst = a.dst.p[s];
      const int64_t row = ((int64_t)b * D + d) * L, t = t0 + 2 * lane;
      if ((L & 1) == 0 && t + 1 < te) {
        if constexpr (IOT == 0) {
          typedef float f32x2v __attribute__((ext_vector_type(2)));
          *reinterpret_cast<f32x2v*>(static_cast<float*>(dst) + row + t) = f32x2v{o0[g], o1[g]};
        } else {
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(dst) + row + t) = bf16x2_bits(o0[g], o1[g]);
        }
      } else {
        if (t < te) st_f<IOT>(dst, row + t, o0[g]);
        if (t + 1 < te) st_f<IOT>(dst, row + t + 1, o1[g]);
      }
    }
  }
}

// ------------------------------------------------------------ in-projection
//
// Workgroup = (batch b, time strip, 128-column block).  The strip's tiles run
// in order; carry[n][j] holds Z row (tile start - HALO + j) of column n.
template <int IOT, bool VEC>
__global__ void __launch_bounds__(TT, 2) k_inproj(InProjArgs a, int n_strips, int strip_len, int n_cb, XcdTiles m) {
  using E = typename Op<IOT>::E;
  constexpr int LDK = Op<IOT>::LDK, BK = Op<IOT>::BK;
  constexpr int MAIN_BYTES = 2 * TM * LDK * (int)sizeof(E);
  constexpr int EPI_BYTES = 64 * ZLD * 4;
  constexpr int BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[BYTES];
  __shared__ float carry[TN][HALO];
  __shared__ float taps[TN][HALO];
  __shared__ float bias[TN];
  E* As = reinterpret_cast<E*>(smem);
  E* Bs = As + TM * LDK;
  float* Zs = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  int job, cb;
  if (!m.tile_of(blockIdx.x, a.B * n_strips, n_cb, job, cb)) return;   // idle slot (whole workgroup)
  const int strip = job % n_strips, b = job / n_strips;
  const int c0 = cb * TN, D = a.D, C = a.C, T = a.T;
  const int64_t L = a.L;
  const int64_t ts = (int64_t)strip * strip_len;
  const int64_t te = (ts + strip_len < L) ? ts + strip_len : L;
  const E* u = static_cast<const E*>(a.u);
  const E* Wt = static_cast<const E*>(a.W);

  // Z rows ts-1 .. ts-(T-1) by direct dot products (zero before t = 0).
  for (int i = tid; i < TN * HALO; i += TT) {
    const int n = i / HALO, j = i % HALO, c = c0 + n;
    (&carry[0][0])[i] = 0.f;
    taps[n][j] = (j < T && c < C) ? a.w[(int64_t)c * T + j] : 0.f;
    if (j == 0) bias[n] = (a.bias && c < C) ? a.bias[c] : 0.f;
  }
  __syncthreads();
  for (int i = tid; i < TN * (T - 1); i += TT) {
    const int n = i % TN, jj = i / TN;               // row ts - 1 - jj
    const int64_t t = ts - 1 - jj;
    const int c = c0 + n;
    if (t >= 0 && c < C) {
      const float z = dot_row<E, VEC>(u + ((int64_t)b * L + t) * D, Wt + (int64_t)c * D, D);
      carry[n][HALO - 1 - jj] = z + (a.bias ? a.bias[c] : 0.f);
    }
  }

  const int nks = (D + BK - 1) / BK;
  const int brhi = (C - c0 < TN) ? C - c0 : TN;
  // The first k-stage of every tile is requested before the previous tile's
  // epilogue, so its loads are not queued behind that epilogue's stores.
  RowStage<IOT, VEC> sa, sb;
  sa.load(u, ((int64_t)b * L + ts) * D, D, (L - ts < TM) ? (int)(L - ts) : TM, 0, D, tid);
  sb.load(Wt, (int64_t)c0 * D, D, brhi, 0, D, tid);
  for (int64_t t0 = ts; t0 < te; t0 += TM) {
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const int64_t aoff = ((int64_t)b * L + t0) * D;
    const int arhi = (L - t0 < TM) ? (int)(L - t0) : TM;
    __syncthreads();                                  // smem free (carry set / last epilogue done)
    sa.store(As, tid);
    sb.store(Bs, tid);
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
      if (ks + 1 < nks) {
        sa.load(u, aoff, D, arhi, (ks + 1) * BK, D, tid);
        sb.load(Wt, (int64_t)c0 * D, D, brhi, (ks + 1) * BK, D, tid);
      }
      Mma<IOT, false>::run(acc, As, Bs, wm, wn, lane);
      __syncthreads();
      if (ks + 1 < nks) {
        sa.store(As, tid);
        sb.store(Bs, tid);
        __syncthreads();
      }
    }
    if (t0 + TM < te) {
      const int64_t t1 = t0 + TM;
      sa.load(u, aoff + (int64_t)TM * D, D, (L - t1 < TM) ? (int)(L - t1) : TM, 0, D, tid);
      sb.load(Wt, (int64_t)c0 * D, D, brhi, 0, D, tid);
    }
    // Epilogue, 64 columns at a time: Z (+bias) and the carried rows into
    // LDS, then the short FIR and the store into the column's stream.
    for (int h = 0; h < 2; ++h) {
      if (h == 1) __syncthreads();                    // half 0's FIR reads done
      if (wn == h) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = j * 32 + (lane & 31);
          const float bc = bias[64 * h + n];   // from LDS: no global load (and wait) in the epilogue
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) Zs[n * ZLD + HALO + wm * 64 + i * 32 + acc_row(r, lane)] = acc[i][j][r] + bc;
        }
      }
      for (int i = tid; i < 64 * HALO; i += TT) {
        const int n = i / HALO, j = i % HALO;
        Zs[n * ZLD + j] = carry[64 * h + n][j];
      }
      __syncthreads();
      // FIR and store: a wave takes columns wave, wave + 4, ... four at a
      // time; lane l makes outputs t0 + 2l and t0 + 2l + 1 of each, so the
      // wave writes every column's 128 outputs as one contiguous run.  The
      // taps beyond T are zero, so K = 4 covers T <= 4 with all loads issued
      // at once.
      if (T <= 4) fir_store<IOT, 4>(a, Zs, taps, h, c0, b, t0, te, wave, lane);
      else fir_store<IOT, HALO>(a, Zs, taps, h, c0, b, t0, te, wave, lane);
      for (int i = tid; i < 64 * HALO; i += TT) {
        const int n = i / HALO, j = i % HALO;
        carry[64 * h + n][j] = Zs[n * ZLD + HALO + TM - HALO + j];
      }
    }
  }
}

// ------------------------------------------- in-projection, bf16 wide tiles
//
// bf16 operands, D a multiple of 8, at most 8 short-filter taps.  Workgroup
// = (batch b, time strip, 256-column block); the strip's tiles of 128 time
// rows run in order.  Wave w owns columns [64w, 64w + 64) of the block at
// all 128 rows of a tile: 4 x 2 accumulator blocks of 32 x 32
// (v_mfma_f32_32x32x16_bf16), so each fragment read from LDS feeds 2 or 4
// MFMAs.  Operand stages of 32 k go from global memory straight into LDS
// (buffer_load_dwordx4 ... lds: no registers, rows outside the data read as
// zero) through a ring of three stage buffers: the loads of stage s + 2 are
// issued as stage s is multiplied, so each has two stages' time to arrive,
// with one barrier per stage.  A stage row is 64 B (4 chunks of 8 bf16);
// chunk q of row r sits at chunk q ^ swz(r) of the row, which spreads both
// the 16-lane and the 8-lane groups of a fragment read over all banks.
//
// The short convolution runs on the accumulators where they are.  Lane l of
// a 32 x 32 block holds column l % 32 at rows 8g + 4(l / 32) + e (g, e < 4):
// read in time order, the block's rows alternate between the two lane
// halves in runs of 4.  One v_permlane32_swap per run position gives each
// half the run before its own, so a lane has its 4 rows and the 4 (or 8)
// before them; rows before a block come from the previous block, and rows
// before a tile from the previous tile of the strip, all kept in registers
// (a wave keeps its columns along the strip).  Each strip starts HALO rows
// early: those rows give the first outputs their history and are not
// stored.  Before t = 0 the rows are zero (no input, no bias).
namespace wide {
constexpr int TM = 128, TN = 256, BK = 32, HALO = 8, NBUF = 3;
constexpr int A_BYTES = TM * BK * 2, B_BYTES = TN * BK * 2, STAGE_BYTES = A_BYTES + B_BYTES;
constexpr uint32_t OOB = 0x80000000u;            // a buffer offset past any record count: reads zero
constexpr int EPI_CS = TM * 2 + 8;                // epilogue column stride in the ring (bytes)
static_assert(4 * 64 * EPI_CS <= NBUF * STAGE_BYTES, "epilogue transpose fits the ring");
// Chunk swizzle of stage row r: 2 bit 2 of r + (bit 1 xor bit 3).  For any
// chunk q, 16 consecutive rows (and 8 consecutive rows) map to 16 (8)
// distinct (r mod 4, q ^ swz) ((r mod 2, q ^ swz)) pairs: distinct banks.
__device__ __forceinline__ int swz(int r) { return (((r >> 2) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1); }
}  // namespace wide

// Workgroup -> (row job, column block) map of the wide in-projection.  The
// 8 XCDs form `groups` groups of 8 / groups XCDs each; group g takes row jobs
// [g * jpg, (g + 1) * jpg) with every column block, and splits those
// (job, block) units, column block slowest, evenly over its XCDs.  An XCD
// then streams the weights of about n_cb * groups / 8 + 1 column blocks
// (few enough to stay in its L2) and shares each input tile among the
// workgroups of its blocks; XCD loads differ by at most one unit.
struct XcdSplit {
  int groups, jpg, per_xcd;
  __device__ __forceinline__ bool tile_of(int w, int jobs, int cbs, int& job, int& cb) const {
    const int x = w & 7, k = w >> 3;
    const int per = 8 / groups, g = x / per, xi = x - g * per;
    const int j0 = g * jpg;
    const int nj = (jobs - j0 < jpg) ? jobs - j0 : jpg;
    if (nj <= 0) return false;
    const int64_t n = (int64_t)nj * cbs;
    const int64_t u = xi * n / per + k;
    if (k >= per_xcd || u >= (xi + 1) * n / per) return false;
    cb = (int)(u / nj);
    job = j0 + (int)(u - (int64_t)cb * nj);
    return true;
  }
};

// The split for `jobs` row jobs x `cbs` column blocks of `block_bytes` of
// weights each: the most groups (least input re-read across XCDs) whose
// weight share per XCD stays within 2.5 MiB of its 4 MiB L2, unless
// HYENA_INPROJ_GROUPS (1, 2, 4 or 8) says otherwise.
static XcdSplit plan_split(int jobs, int cbs, int64_t block_bytes, int64_t& grid) {
  int groups = 1;
  for (int g = 8; g >= 1; g /= 2) {
    const int64_t span = ((int64_t)cbs * g + 7) / 8 + 1;
    if (span * block_bytes <= (int64_t)5 << 19 || g == 1) { groups = g; break; }
  }
  if (const char* e = getenv("HYENA_INPROJ_GROUPS")) {
    const int v = atoi(e);
    if (v == 1 || v == 2 || v == 4 || v == 8) groups = v;
  }
  const int per = 8 / groups;
  const int jpg = ceil_div(jobs, groups);
  const int per_xcd = ceil_div((int64_t)jpg * cbs, per);
  grid = 8LL * per_xcd;
  return XcdSplit{groups, jpg, per_xcd};
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Stage loads of one workgroup: A (128 time rows) is 8 instructions of 64
// chunks, 2 per wave; B (256 columns) is 16, 4 per wave.  Instruction j of
// wave w fills stage slots [64 (J w + j), +64) in lane order, so each lane
// fetches the chunk that belongs in its slot: row s / 4, chunk (s % 4) ^
// swz(row).  off: byte offset of (row, chunk) from the resource base, OOB
// for rows outside the data; kq: the chunk's k offset (8 chunk).
template <int J>
struct WideLoads {
  uint32_t off[J];
  int kq[J];
  // Stage at k0.  exact: D is a multiple of the stage depth, so every chunk
  // of a row in the data is inside it and k0 goes in the scalar offset.
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, unsigned char* dst, int w, int k0, int D,
                                        bool exact) const {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      lds_ptr_t d = (lds_ptr_t)(dst + (J * w + j) * 1024);
      if (exact) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, (int)off[j], 2 * k0, 0, 0);
      } else {
        const uint32_t o = (k0 + kq[j] < D && off[j] != wide::OOB) ? off[j] + 2u * (uint32_t)k0 : wide::OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, (int)o, 0, 0, 0);
      }
    }
  }
};

template <int KT, bool AL8>
__global__ void __launch_bounds__(256, 2) k_inproj_wide(InProjArgs a, int n_strips, int64_t strip_len, int n_cb,
                                                       XcdSplit m) {
  constexpr int TM = wide::TM, TN = wide::TN, BK = wide::BK, HALO = wide::HALO, NB = wide::NBUF;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NB * wide::STAGE_BYTES];
  __shared__ uint16_t* colp[TN];                    // output row of each column of the block (null past C)
  static_assert(HALO == 8, "the strip at t = 0 starts one run pair early");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  int job, cb;
  if (!m.tile_of(blockIdx.x, a.B * n_strips, n_cb, job, cb)) return;   // idle slot (whole workgroup)
  const int strip = job % n_strips, b = job / n_strips;
  const int D = a.D, C = a.C, T = a.T, c0 = cb * TN;
  const int64_t L = a.L;
  const int64_t ts = (int64_t)strip * strip_len;
  const int64_t te = (ts + strip_len < L) ? ts + strip_len : L;
  const uint16_t* u = static_cast<const uint16_t*>(a.u) + (int64_t)b * L * D;

  // This lane's two columns: taps, bias and bias * sum of taps; the
  // block's output rows.
  float tap[2][KT], bias[2], bsum[2];
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int c = c0 + 64 * w + 32 * jb + l32;
    const bool ok = c < C;
    float ts_ = 0.f;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      tap[jb][j] = (ok && j < T) ? a.w[(int64_t)c * T + j] : 0.f;
      ts_ += tap[jb][j];
    }
    bias[jb] = (ok && a.bias) ? a.bias[c] : 0.f;
    bsum[jb] = bias[jb] * ts_;
  }
  {
    const int c = c0 + tid;
    colp[tid] = c < C ? static_cast<uint16_t*>(a.dst.p[c / D]) + ((int64_t)b * D + c % D) * L : nullptr;
  }

  // B (the block's weight rows) for the whole strip.
  const int nb_rows = (C - c0 < TN) ? C - c0 : TN;
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(static_cast<const uint16_t*>(a.W) + (int64_t)c0 * D), (short)0, nb_rows * D * 2, 0x00020000);
  WideLoads<4> lb;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sl = (4 * w + j) * 64 + lane, r = sl >> 2, q = (sl & 3) ^ wide::swz(r);
    lb.kq[j] = 8 * q;
    lb.off[j] = r < nb_rows ? (uint32_t)(r * D + 8 * q) * 2u : wide::OOB;
  }

  // Fragment reads: row l32 of a 32-row block, chunk (2 kk + h) ^ swz(l32).
  const int fsw = wide::swz(l32);
  const int fo0 = l32 * 64 + 16 * (h ^ fsw), fo1 = l32 * 64 + 16 * ((2 + h) ^ fsw);

  float xp[2][4];                                    // the run pair before the current one (Z, both halves)
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int e = 0; e < 4; ++e) xp[jb][e] = 0.f;

  const int nks = (D + BK - 1) / BK;
  __amdgpu_buffer_rsrc_t rsa;
  WideLoads<2> la;
  // A of the tile at rows [t0, t0 + TM): resource from the first row >= 0.
  auto tile_a = [&](int64_t t0) {
    const int64_t tlo = t0 > 0 ? t0 : 0, thi = (t0 + TM < L) ? t0 + TM : L;
    const int nrows = thi > tlo ? (int)(thi - tlo) : 0;
    rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(u + tlo * D), (short)0, nrows * D * 2, 0x00020000);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int sl = (2 * w + j) * 64 + lane, r = sl >> 2, q = (sl & 3) ^ wide::swz(r);
      const int64_t t = t0 + r;
      la.kq[j] = 8 * q;
      la.off[j] = (t >= tlo && t < thi) ? (uint32_t)((t - tlo) * D + 8 * q) * 2u : wide::OOB;
    }
  };
  const bool exact = D % BK == 0;
  auto issue = [&](int ks) {
    unsigned char* st = lds + (ks % NB) * wide::STAGE_BYTES;
    la.issue(rsa, st, w, ks * BK, D, exact);
    lb.issue(rsb, st + wide::A_BYTES, w, ks * BK, D, exact);
  };

  int64_t t0 = ts - HALO;
  tile_a(t0);
  issue(0);
  if (nks > 1) issue(1);
  for (; t0 < te; t0 += TM) {
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][jb][r] = 0.f;

    for (int ks = 0; ks < nks; ++ks) {
      // This wave's loads of stage ks are done once at most those of stage
      // ks + 1 (6 instructions) are outstanding; its reads of the buffer
      // refilled below are done; the barrier makes both hold for all waves.
      if (ks + 1 < nks) __builtin_amdgcn_s_waitcnt(0x0076);     // vmcnt(6) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(0x0070);                  // vmcnt(0) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (ks + 2 < nks) issue(ks + 2);
      const unsigned char* As = lds + (ks % NB) * wide::STAGE_BYTES;
      const unsigned char* Bs = As + wide::A_BYTES + 64 * 64 * w;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int fo = kk ? fo1 : fo0;
        bf16x8 fa[4], fb[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(As + 32 * 64 * i + fo);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) fb[jb] = *reinterpret_cast<const bf16x8*>(Bs + 32 * 64 * jb + fo);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jb = 0; jb < 2; ++jb)
            acc[i][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[jb], acc[i][jb], 0, 0, 0);
      }
    }
    // Every wave's reads of the ring are done: it is free for the epilogue.
    __builtin_amdgcn_s_waitcnt(0xc07f);                         // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

    // Short convolution, one run pair (8 rows) at a time, into this wave's
    // part of the idle ring as [column][time] bf16 (column stride 264 B:
    // the 32 columns of a half-wave write fall on distinct banks); then each
    // 16 lanes store one column's 128 outputs, 256 B.  The bias enters once
    // per output as bias * (sum of the taps): the convolution runs on the
    // products alone, which are zero before t = 0, and the first KT - 1
    // outputs (t < KT - 1) drop the taps that reach before t = 0.
    unsigned char* ep = lds + w * 64 * wide::EPI_CS;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = k >> 2, g = k & 3;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        float x[4], y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[i][jb][4 * g + e];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (KT <= 4 && e < 5 - KT) { y[e] = 0.f; continue; }   // not reached by KT taps
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(xp[jb][e]), __float_as_uint(x[e]), false,
                                                           false);
          y[e] = __uint_as_float(h ? sw[0] : sw[1]);
        }
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float s = bsum[jb];
#pragma unroll
          for (int j = 0; j < KT; ++j) {
            const int d = e - j;
            const float z = d >= 0 ? x[d] : (d >= -4 ? y[d + 4] : xp[jb][d + 8]);
            s = fmaf(tap[jb][j], z, s);
          }
          o[e] = s;
        }
        if (k == HALO / 8 && t0 < 0) {               // the strip at t = 0: rows t0 + 8k + 4h + e = 4h + e
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int j = 1; j < KT; ++j)
              if (4 * h + e < j) o[e] = fmaf(-bias[jb], tap[jb][j], o[e]);
        }
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x2*>(ep + (32 * jb + l32) * wide::EPI_CS + (8 * k + 4 * h) * 2) =
            u32x2{bf16x2_bits(o[0], o[1]), bf16x2_bits(o[2], o[3])};
#pragma unroll
        for (int e = 0; e < 4; ++e) xp[jb][e] = x[e];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
      const int ch = lane & 15;                      // 8 outputs t0 + 8 ch .. + 7 of the column
      const int64_t tc = t0 + 8 * ch;
#pragma unroll 4
      for (int q = 0; q < 16; ++q) {
        const int col = 4 * q + (lane >> 4);
        const u32x4 v = *reinterpret_cast<const u32x4*>(ep + col * wide::EPI_CS + 16 * ch);
        uint16_t* p = colp[64 * w + col];
        if (!p) continue;
        if (AL8 && tc >= ts && tc + 8 <= te) {
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p + tc));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (tc + e >= ts && tc + e < te) p[tc + e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
    // Every wave is done with the ring: the next tile's first stages may load.
    __builtin_amdgcn_s_waitcnt(0xc07f);                         // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (t0 + TM < te) {
      tile_a(t0 + TM);
      issue(0);
      if (nks > 1) issue(1);
    }
  }
}

// ----------------------------------------------------------- out-projection
//
// Workgroup = (batch b, 128 time rows, 128 output columns).  A = y^T: the
// stage reads y rows (one channel, consecutive times); fp32 keeps them
// k-major in LDS, bf16 transposes them to [time][channel] for the MFMA's
// 8-consecutive-k operand.
template <int IOT, bool VEC>
struct YStage {
  using E = typename Op<IOT>::E;
  static constexpr int W = Op<IOT>::W;
  u32x4 v[4];
  // fp32 item: k = idx >> 5 (32 channels), 4 times; bf16 item: k = idx & 63, 8 times
  __device__ __forceinline__ void load(const E* y, int64_t ybase, int64_t L, int D, int d0, int64_t t0, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + TT * i;
      const int k = (IOT == 0) ? (idx >> 5) : (idx & 63);
      const int q = (IOT == 0) ? (idx & 31) : (idx >> 6);
      const int d = d0 + k;
      const int64_t t = t0 + (int64_t)q * W;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (d < D && t < L) {
        const E* p = y + ybase + (int64_t)d * L + t;
        if constexpr (VEC) {
          w = *reinterpret_cast<const u32x4*>(p);
        } else if constexpr (IOT == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (t + e < L) ? __float_as_uint(p[e]) : 0u;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (t + e < L) w[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
        }
      }
      v[i] = w;
    }
  }
  __device__ __forceinline__ void store(E* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + TT * i;
      if constexpr (IOT == 0) {
        const int k = idx >> 5, q = (idx & 31) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) lds[k * (TM + 4) + q + e] = __uint_as_float(v[i][e]);
      } else {
        const int k = idx & 63, q = (idx >> 6) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) lds[(q + e) * Op<1>::LDK + k] = (uint16_t)(v[i][e >> 1] >> (16 * (e & 1)));
      }
    }
  }
};

template <int IOT, bool VEC>
__global__ void __launch_bounds__(TT, 2) k_outproj(OutProjArgs a, int n_tt, int n_eb, XcdTiles m) {
  using E = typename Op<IOT>::E;
  constexpr int LDK = Op<IOT>::LDK, BK = Op<IOT>::BK;
  constexpr int A_ELEMS = (IOT == 0) ? BK * (TM + 4) : TM * LDK;
  __shared__ __attribute__((aligned(16))) E As[A_ELEMS];
  __shared__ __attribute__((aligned(16))) E Bs[TN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  int job, eb;
  if (!m.tile_of(blockIdx.x, a.B * n_tt, n_eb, job, eb)) return;       // idle slot (whole workgroup)
  const int tt = job % n_tt, b = job / n_tt;
  const int D = a.D, e0 = eb * TN;
  const int64_t L = a.L, t0 = (int64_t)tt * TM;
  const E* y = static_cast<const E*>(a.y);
  const E* Wt = static_cast<const E*>(a.W);
  const int64_t ybase = (int64_t)b * D * L;
  const int brhi = (D - e0 < TN) ? D - e0 : TN;
  const int nks = (D + BK - 1) / BK;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  YStage<IOT, VEC> sa;
  RowStage<IOT, VEC> sb;
  sa.load(y, ybase, L, D, 0, t0, tid);
  sb.load(Wt, (int64_t)e0 * D, D, brhi, 0, D, tid);
  sa.store(As, tid);
  sb.store(Bs, tid);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    if (ks + 1 < nks) {
      sa.load(y, ybase, L, D, (ks + 1) * BK, t0, tid);
      sb.load(Wt, (int64_t)e0 * D, D, brhi, (ks + 1) * BK, D, tid);
    }
    Mma<IOT, IOT == 0>::run(acc, As, Bs, wm, wn, lane);
    __syncthreads();
    if (ks + 1 < nks) {
      sa.store(As, tid);
      sb.store(Bs, tid);
      __syncthreads();
    }
  }
  void* out = a.out;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + wn * 64 + j * 32 + (lane & 31);
    const bool ev = e < D;
    // the bias is read outside the stores' lane masks and pinned: read
    // inside them, every masked store would first wait for all earlier
    // stores (the memory counter tracks both)
    float be = a.bias ? a.bias[ev ? e : 0] : 0.f;
    asm volatile("" : "+v"(be));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = t0 + wm * 64 + i * 32 + acc_row(r, lane);
        if (ev && t < L) st_f<IOT>(out, ((int64_t)b * L + t) * D + e, acc[i][j][r] + be);
      }
  }
}

template <int IOT, bool VEC>
static hipError_t launch_inproj(const InProjArgs& a, hipStream_t s) {
  const auto kern = k_inproj<IOT, VEC>;
  const int n_cb = ceil_div(a.C, TN);
  const int tiles = ceil_div(a.L, TM);
  // Workgroups run whole strips of tiles, so they are long-lived: at most as
  // many as fit the GPU at once, never a second partial wave.
  int dev = 0, cus = 256, per_cu = 1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, TT, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t cap = (int64_t)cus * per_cu;
  int want = (int)(cap / ((int64_t)a.B * n_cb));
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  int n_strips, per;
  int64_t grid = 0;
  XcdTiles m;
  for (;; --want) {                 // fewer strips until the mapped grid fits at once
    per = ceil_div(tiles, want);
    n_strips = ceil_div(tiles, per);
    m = plan_xcd(a.B * n_strips, n_cb, grid);
    if (grid <= cap || want == 1) break;
  }
  const int strip_len = per * TM;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(TT), 0, s, a, n_strips, strip_len, n_cb, m);
  return hipGetLastError();
}

// Strips of whole tiles (the first HALO rows of each are history only), as
// many as fit the GPU at once after the XCD map.
template <int KT, bool AL8>
static hipError_t launch_inproj_wide(const InProjArgs& a, hipStream_t s) {
  const auto kern = k_inproj_wide<KT, AL8>;
  const int n_cb = ceil_div(a.C, wide::TN);
  int dev = 0, cus = 256, per_cu = 1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t cap = (int64_t)cus * per_cu;
  const int64_t max_tiles = (a.L + wide::HALO + wide::TM - 1) / wide::TM;
  const int64_t block_bytes = (int64_t)wide::TN * a.D * 2;
  int64_t grid = 0, strip_len = 0;
  int n_strips = 0;
  XcdSplit m{};
  int64_t per0 = max_tiles * a.B * n_cb / cap;   // fewer tiles per strip cannot fit
  if (per0 < 1) per0 = 1;
  for (int64_t per = per0;; ++per) {     // tiles per strip: the fewest whose grid fits at once
    strip_len = per * wide::TM - wide::HALO;
    const int64_t ns = (a.L + strip_len - 1) / strip_len;
    if ((int64_t)a.B * ns > (1LL << 30)) continue;
    n_strips = (int)ns;
    m = plan_split(a.B * n_strips, n_cb, block_bytes, grid);
    if (grid <= cap || per >= max_tiles) break;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, a, n_strips, strip_len, n_cb, m);
  return hipGetLastError();
}

}  // namespace

hipError_t in_projection(const InProjArgs& a, hipStream_t s) {
  if (a.io == 1 && a.D % 8 == 0 && a.T <= 8) {
    const bool al8 = a.L % 8 == 0;
    switch (a.T <= 2 ? 2 : a.T <= 4 ? a.T : 8) {
      case 2: return al8 ? launch_inproj_wide<2, true>(a, s) : launch_inproj_wide<2, false>(a, s);
      case 3: return al8 ? launch_inproj_wide<3, true>(a, s) : launch_inproj_wide<3, false>(a, s);
      case 4: return al8 ? launch_inproj_wide<4, true>(a, s) : launch_inproj_wide<4, false>(a, s);
      default: return al8 ? launch_inproj_wide<8, true>(a, s) : launch_inproj_wide<8, false>(a, s);
    }
  }
  const bool vec = a.D % (a.io == 0 ? 4 : 8) == 0;
  if (a.io == 0) return vec ? launch_inproj<0, true>(a, s) : launch_inproj<0, false>(a, s);
  return vec ? launch_inproj<1, true>(a, s) : launch_inproj<1, false>(a, s);
}

hipError_t out_projection(const OutProjArgs& a, hipStream_t s) {
  const int n_eb = ceil_div(a.D, TN), n_tt = ceil_div(a.L, TM);
  int64_t g = 0;
  const XcdTiles m = plan_xcd(a.B * n_tt, n_eb, g);
  const dim3 grid((unsigned)g), block(TT);
  const int w = (a.io == 0 ? 4 : 8);
  const bool vec = a.D % w == 0 && a.L % w == 0;
  if (a.io == 0) {
    if (vec) hipLaunchKernelGGL((k_outproj<0, true>), grid, block, 0, s, a, n_tt, n_eb, m);
    else hipLaunchKernelGGL((k_outproj<0, false>), grid, block, 0, s, a, n_tt, n_eb, m);
  } else {
    if (vec) hipLaunchKernelGGL((k_outproj<1, true>), grid, block, 0, s, a, n_tt, n_eb, m);
    else hipLaunchKernelGGL((k_outproj<1, false>), grid, block, 0, s, a, n_tt, n_eb, m);
  }
  return hipGetLastError();
}

}  // namespace hyena
