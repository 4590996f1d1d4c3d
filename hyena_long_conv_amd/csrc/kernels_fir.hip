// kernels_fir.hip -- the other filter families of homemade-llm "02. 3つの
// Hyena 演算子", section 3: Hyena-LI filters (a sum of real exponentials per
// filter, fed to the FFT path), Hyena-MR damping of explicit filters, and the
// order-N recurrence with explicit short filters (Hyena-SE, Hyena-MR)
// evaluated directly, the causal FIR of the same page's section 4.
#include <hip/hip_runtime.h>

#include "fft_engine.hpp"
#include "launch.hpp"

namespace hyena {
namespace {

// h[f][t] = sum_s R[f][s] * lambda[f][s]^t, in double (exponents up to 4M).
__global__ void k_filter_gen_li(const float* __restrict__ R, const float* __restrict__ lam, int S, int64_t L,
                                int64_t total, float* __restrict__ h) {
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t f = idx / L, t = idx - f * L;
    double acc = 0.0;
    for (int s = 0; s < S; ++s) {
      const double r = R[f * S + s], l = lam[f * S + s];
      double p;
      if (t == 0) {
        p = 1.0;
      } else if (l == 0.0) {
        p = 0.0;
      } else {
        p = exp2((double)t * log2(fabs(l)));
        if (l < 0.0 && (t & 1)) p = -p;
      }
      acc += r * p;
    }
    h[idx] = (float)acc;
  }
}

// h[n][d][t] = hhat[n][d][t] * exp(-alpha[d] * t), t < Lh.
__global__ void k_filter_gen_mr(const float* __restrict__ hhat, const float* __restrict__ alpha, int D, int Lh,
                                int64_t total, float* __restrict__ h) {
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t f = idx / Lh, t = idx - f * Lh;
    const int d = (int)(f % D);
    h[idx] = (float)((double)hhat[idx] * exp(-(double)alpha[d] * (double)t));
  }
}

// Recurrence with explicit filters of Lh taps.  Workgroup = (row, time tile
// of TT samples).  z_1 = v is staged over the tile plus a halo of
// N*(Lh-1) earlier samples (zero before t = 0); each order consumes Lh-1 of
// the halo, so after N orders exactly the tile remains, with nothing read
// from other tiles.  Two LDS buffers alternate between orders.  A thread
// computes FR = 4 consecutive outputs, taking the taps four at a time: one
// 16-byte LDS read of the next four window samples, one broadcast 16-byte
// read of four taps, 16 FMAs.  Taps are stored per order in rows of Lh4 =
// Lh rounded up to 4 (zero beyond Lh), and each buffer has PAD zeroed
// floats before it for the window reads left of the first output.
constexpr int FIR_THREADS = 256, FR = 4, PAD = 8, FIR_UNROLL = 3, FIR_BATCH_TAPS = 32;
typedef float fir_f4 __attribute__((ext_vector_type(4)));

template <int IOT>
__device__ __forceinline__ void ld4(const void* p, int64_t i, float (&o)[4]) {   // i a multiple of 4, in range
  if constexpr (IOT == 0) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 w = __builtin_nontemporal_load(reinterpret_cast<const f4*>(static_cast<const float*>(p) + i));
    o[0] = w.x; o[1] = w.y; o[2] = w.z; o[3] = w.w;
  } else {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 w = __builtin_nontemporal_load(reinterpret_cast<const u2*>(static_cast<const uint16_t*>(p) + i));
    o[0] = __uint_as_float(w.x << 16); o[1] = __uint_as_float(w.x & 0xffff0000u);
    o[2] = __uint_as_float(w.y << 16); o[3] = __uint_as_float(w.y & 0xffff0000u);
  }
}

// Windows x[t_u .. t_u+3] (t_u = t + u * STEP, multiples of 4) for u <
// FIR_UNROLL, zero outside [0, L).  Rows of a length that is a multiple of 4
// (vec): every window is one aligned access from a clamped index (a window is
// then all in or all out of the row), all issued before any is masked, so no
// branch separates them: a load inside a lane-masked branch is waited for
// before the next is issued.  Other rows go sample by sample.
template <int IOT>
__device__ __forceinline__ void ld4_batch(const void* p, int64_t off, int64_t t, int64_t L, bool vec,
                                          float (&o)[FIR_UNROLL][4]) {
  constexpr int STEP = 4 * FIR_THREADS;
  if (vec) {
#pragma unroll
    for (int u = 0; u < FIR_UNROLL; ++u) {
      const int64_t tu = t + u * STEP;
      ld4<IOT>(p, off + (tu < 0 ? 0 : (tu >= L ? L - 4 : tu)), o[u]);
    }
#pragma unroll
    for (int u = 0; u < FIR_UNROLL; ++u) {
      const int64_t tu = t + u * STEP;
      const bool in = tu >= 0 && tu < L;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[u][q] = in ? o[u][q] : 0.f;
    }
  } else {
#pragma unroll
    for (int u = 0; u < FIR_UNROLL; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t tq = t + u * STEP + q;
        o[u][q] = (tq >= 0 && tq < L) ? IO<IOT>::ld(p, off + tq) : 0.f;
      }
  }
}

template <int IOT>
__global__ void __launch_bounds__(FIR_THREADS) k_fir_forward(const void* __restrict__ v, XPtrs x,
                                                              const float* __restrict__ h, int Lh,
                                                              void* __restrict__ y, int D, int NORD, int64_t L,
                                                              int TT) {
  extern __shared__ float sm[];
  const int row = blockIdx.x, d = row % D;
  const int64_t t0 = (int64_t)blockIdx.y * TT;
  const int Hh = (NORD * (Lh - 1) + 3) / 4 * 4;  // halo, a multiple of 4 (extra samples are harmless)
  const int W = TT + Hh;                         // buffer index i <-> time t0 - Hh + i
  const int Lh4 = (Lh + 3) / 4 * 4;
  float* b0 = sm + PAD;
  float* b1 = sm + 2 * PAD + W;
  float* taps = sm + 2 * (PAD + W);
  const int64_t off = (int64_t)row * L;
  const int tid = threadIdx.x;
  const bool vec = (L & 3) == 0;                 // rows start on 16-byte (fp32) / 8-byte (bf16) boundaries
  if (tid < 2 * PAD) sm[tid < PAD ? tid : W + tid] = 0.f;   // the two pads
  for (int i = tid; i < NORD * Lh4; i += FIR_THREADS) {
    const int n = i / Lh4, k = i - n * Lh4;
    taps[i] = k < Lh ? h[((int64_t)n * D + d) * Lh + k] : 0.f;
  }
  // Windows of 4 samples, FIR_UNROLL passes of the workgroup at a time: the
  // loads of a batch are issued together (from in-row addresses, also on
  // lanes past the end, which store nothing), then stored.
  constexpr int STEP = 4 * FIR_THREADS;
  for (int c0 = 0; c0 * STEP < W; c0 += FIR_UNROLL) {
    float o[FIR_UNROLL][4];
    ld4_batch<IOT>(v, off, t0 - Hh + 4 * tid + c0 * STEP, L, vec, o);
#pragma unroll
    for (int u = 0; u < FIR_UNROLL; ++u) {
      const int i4 = 4 * tid + (c0 + u) * STEP;
      if (i4 < W) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          b0[i4 + q] = o[u][q];
          b1[i4 + q] = 0.f;   // an order writes b1 from its first full-history output on; the
        }                     // rest must hold finite values, since zero taps beyond Lh still read it
      }
    }
  }
  __syncthreads();
  for (int n = 0; n < NORD; ++n) {
    const int lo = (n + 1) * (Lh - 1);           // first index with a full history
    const int lo4 = lo / 4 * 4;
    const float* tp = taps + n * Lh4;
    const void* xn = x.p[n];
    // outputs i0 .. i0+3: acc[r] = sum_k h[k] b0[i0 + r - k].  For the taps
    // k0 .. k0+3, cur = b0[i0-k0 .. i0-k0+3] and prv = the four before it
    // (the lowest read is i0 - Lh4 >= -7, inside the pad).
    const auto fir4 = [&](int i0, const float* xv) {
      float acc[FR] = {0.f, 0.f, 0.f, 0.f};
      fir_f4 cur = *reinterpret_cast<const fir_f4*>(b0 + i0);
      for (int k0 = 0; k0 < Lh4; k0 += 4) {
        const fir_f4 prv = *reinterpret_cast<const fir_f4*>(b0 + i0 - k0 - 4);
        const fir_f4 hv = *reinterpret_cast<const fir_f4*>(tp + k0);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int r = 0; r < FR; ++r) acc[r] = fmaf(hv[m], r >= m ? cur[r - m] : prv[4 + r - m], acc[r]);
        cur = prv;
      }
#pragma unroll
      for (int r = 0; r < FR; ++r) b1[i0 + r] = xv[r] * acc[r];
    };
    if (Lh4 <= FIR_BATCH_TAPS) {
      // short filters: the sums are short next to a memory round trip, so the
      // gates of FIR_UNROLL passes are requested together before them
      for (int c0 = 0; lo4 + c0 * STEP < W; c0 += FIR_UNROLL) {
        float xb[FIR_UNROLL][4];
        ld4_batch<IOT>(xn, off, t0 - Hh + lo4 + FR * tid + c0 * STEP, L, vec, xb);
#pragma unroll
        for (int u = 0; u < FIR_UNROLL; ++u) {
          const int i0 = lo4 + FR * tid + (c0 + u) * STEP;
          if (i0 < W) fir4(i0, xb[u]);
        }
      }
    } else {
      for (int i0 = lo4 + FR * tid; i0 < W; i0 += STEP) {
        const int64_t t = t0 - Hh + i0;
        float xv[4];
        if (vec && t >= 0 && t + 3 < L) {
          ld4<IOT>(xn, off + t, xv);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) xv[q] = (t + q >= 0 && t + q < L) ? IO<IOT>::ld(xn, off + t + q) : 0.f;
        }
        fir4(i0, xv);
      }
    }
    __syncthreads();
    float* tmp = b0;
    b0 = b1;
    b1 = tmp;
  }
  for (int i4 = Hh + 4 * tid; i4 < W; i4 += 4 * FIR_THREADS) {
    const int64_t t = t0 - Hh + i4;
    if (vec && t + 3 < L) {
      if constexpr (IOT == 0) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4 w = {b0[i4], b0[i4 + 1], b0[i4 + 2], b0[i4 + 3]};
        __builtin_nontemporal_store(w, reinterpret_cast<f4*>(static_cast<float*>(y) + off + t));
      } else {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 w = {bf16x2_bits(b0[i4], b0[i4 + 1]), bf16x2_bits(b0[i4 + 2], b0[i4 + 3])};
        __builtin_nontemporal_store(w, reinterpret_cast<u2*>(static_cast<uint16_t*>(y) + off + t));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (t + q < L) IO<IOT>::st(y, off + t + q, b0[i4 + q]);
    }
  }
}

}  // namespace

hipError_t filter_gen_li(const float* R, const float* lam, int NF, int S, int64_t L, float* h, hipStream_t s) {
  const int64_t total = (int64_t)NF * L;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_filter_gen_li, dim3((unsigned)(blocks < 65536 * 8 ? blocks : 65536 * 8)), dim3(256), 0, s,
                     R, lam, S, L, total, h);
  return hipGetLastError();
}

hipError_t filter_gen_mr(const float* hhat, const float* alpha, int D, int NF, int Lh, float* h, hipStream_t s) {
  const int64_t total = (int64_t)NF * Lh;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_filter_gen_mr, dim3((unsigned)(blocks < 65536 * 8 ? blocks : 65536 * 8)), dim3(256), 0, s,
                     hhat, alpha, D, Lh, total, h);
  return hipGetLastError();
}

hipError_t fir_forward(const ForwardArgs& a, const float* h, int Lh, hipStream_t s) {
  const int TT = 2048;
  const int64_t tiles = (a.L + TT - 1) / TT;
  const int halo = (a.NORD * (Lh - 1) + 3) / 4 * 4;
  const size_t lds = (size_t)(2 * (PAD + TT + halo) + a.NORD * ((Lh + 3) / 4 * 4)) * sizeof(float);
  const dim3 grid((unsigned)a.n_rows, (unsigned)tiles), block(FIR_THREADS);
  if (a.io == 0)
    hipLaunchKernelGGL(k_fir_forward<0>, grid, block, lds, s, a.v, a.x, h, Lh, a.y, a.D, a.NORD, a.L, TT);
  else
    hipLaunchKernelGGL(k_fir_forward<1>, grid, block, lds, s, a.v, a.x, h, Lh, a.y, a.D, a.NORD, a.L, TT);
  return hipGetLastError();
}

}  // namespace hyena
