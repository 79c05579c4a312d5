// The identity-map step as one flat stream: M <- beta M + G (one fp32 fused multiply-add,
// stored in the state dtype with RNE) and W <- W - lr M over n contiguous elements, with
// no tiling.  It moves exactly the bytes of the tiled step's memory pass (G and M read, M
// written, W read and written), so its rate is the HBM rate this read/write mix allows on
// the device: the reference for the memory pass of the fused kernel.
#include "device_common.h"
#include "himuon_internal.h"

namespace himuon {
namespace {

using namespace dev;

constexpr int STREAM_THREADS = 256;

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// VEC: m, g and w are 16-byte aligned; each thread takes 8 consecutive elements per turn
// (16-byte loads and stores of the state, two of W), the last n % 8 go element by element.
template <typename S, bool VEC>
__global__ __launch_bounds__(STREAM_THREADS) void stream_step_kernel(S *__restrict__ m, const S *__restrict__ g,
                                                                     float *__restrict__ w, int64_t n, float beta,
                                                                     float lr) {
  const int64_t tid = (int64_t)blockIdx.x * STREAM_THREADS + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * STREAM_THREADS;
  const float nlr = -lr;
  int64_t done = 0;
  if constexpr (VEC) {
    const int64_t n8 = n / 8;
    for (int64_t i = tid; i < n8; i += nthreads) {
      float v[8];
      if constexpr (sizeof(S) == 2) {
        const u32x4 gv = gmem(reinterpret_cast<const u32x4 *>(g))[i];
        const u32x4 mv = gmem(reinterpret_cast<const u32x4 *>(m))[i];
        u32x4 code;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          code[e] = pack_bf16x2(__builtin_fmaf(beta, bf16_lo(mv[e]), bf16_lo(gv[e])),
                                __builtin_fmaf(beta, bf16_hi(mv[e]), bf16_hi(gv[e])));
          v[2 * e] = bf16_lo(code[e]);
          v[2 * e + 1] = bf16_hi(code[e]);
        }
        gmem(reinterpret_cast<u32x4 *>(m))[i] = code;
      } else {
        const f32x4 g0 = gmem(reinterpret_cast<const f32x4 *>(g))[2 * i], g1 = gmem(reinterpret_cast<const f32x4 *>(g))[2 * i + 1];
        const f32x4 m0 = gmem(reinterpret_cast<const f32x4 *>(m))[2 * i], m1 = gmem(reinterpret_cast<const f32x4 *>(m))[2 * i + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = __builtin_fmaf(beta, m0[e], g0[e]);
          v[e + 4] = __builtin_fmaf(beta, m1[e], g1[e]);
        }
        gmem(reinterpret_cast<f32x4 *>(m))[2 * i] = f32x4{v[0], v[1], v[2], v[3]};
        gmem(reinterpret_cast<f32x4 *>(m))[2 * i + 1] = f32x4{v[4], v[5], v[6], v[7]};
      }
      const f32x4 w0 = gmem(reinterpret_cast<const f32x4 *>(w))[2 * i], w1 = gmem(reinterpret_cast<const f32x4 *>(w))[2 * i + 1];
      gmem(reinterpret_cast<f32x4 *>(w))[2 * i] =
          f32x4{__builtin_fmaf(nlr, v[0], w0[0]), __builtin_fmaf(nlr, v[1], w0[1]), __builtin_fmaf(nlr, v[2], w0[2]),
                __builtin_fmaf(nlr, v[3], w0[3])};
      gmem(reinterpret_cast<f32x4 *>(w))[2 * i + 1] =
          f32x4{__builtin_fmaf(nlr, v[4], w1[0]), __builtin_fmaf(nlr, v[5], w1[1]), __builtin_fmaf(nlr, v[6], w1[2]),
                __builtin_fmaf(nlr, v[7], w1[3])};
    }
    done = n8 * 8;
  }
  for (int64_t k = done + tid; k < n; k += nthreads) {
    float v;
    if constexpr (sizeof(S) == 2) {
      const unsigned short gb = gmem(reinterpret_cast<const unsigned short *>(g))[k];
      const unsigned short mb = gmem(reinterpret_cast<const unsigned short *>(m))[k];
      const unsigned short code = to_bf16_bits(
          __builtin_fmaf(beta, __builtin_bit_cast(float, (unsigned)mb << 16), __builtin_bit_cast(float, (unsigned)gb << 16)));
      gmem(reinterpret_cast<unsigned short *>(m))[k] = code;
      v = __builtin_bit_cast(float, (unsigned)code << 16);
    } else {
      v = __builtin_fmaf(beta, gmem(m)[k], gmem(g)[k]);
      gmem(m)[k] = v;
    }
    gmem(w)[k] = __builtin_fmaf(nlr, v, gmem(w)[k]);
  }
}

template <typename S>
hipError_t launch_stream_t(void *m, const void *g, float *w, int64_t n, float beta, float lr, hipStream_t stream) {
  const bool vec = ((reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(w)) & 15) == 0;
  const int64_t work = vec ? (n + 7) / 8 : n;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((work + STREAM_THREADS - 1) / STREAM_THREADS, 16384));
  if (vec)
    hipLaunchKernelGGL((stream_step_kernel<S, true>), dim3((unsigned)blocks), dim3(STREAM_THREADS), 0, stream,
                       reinterpret_cast<S *>(m), reinterpret_cast<const S *>(g), w, n, beta, lr);
  else
    hipLaunchKernelGGL((stream_step_kernel<S, false>), dim3((unsigned)blocks), dim3(STREAM_THREADS), 0, stream,
                       reinterpret_cast<S *>(m), reinterpret_cast<const S *>(g), w, n, beta, lr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_step(void *m, const void *g, float *w, int64_t n, bool state_bf16, float beta, float lr,
                              hipStream_t stream) {
  return state_bf16 ? launch_stream_t<__bf16>(m, g, w, n, beta, lr, stream)
                    : launch_stream_t<float>(m, g, w, n, beta, lr, stream);
}

}  // namespace himuon
