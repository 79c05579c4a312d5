// Sign-Muon's local kernels ("Sign-Muon: Communication-Efficient Distributed Muon
// Optimization", Figures 1 and 6): the entrywise sign of a direction matrix packed to one
// bit per entry, and the majority vote over the packed buffers of several workers.
//
// Packing: entry k = i * cols + j of a rows x cols matrix (row-major, any leading
// dimension) is bit k % 8 of byte k / 8, 1 for +1; sign(0) = +1 (and sign(NaN) = -1, as
// the comparison x >= 0 is false for it).  Each wave takes 64 consecutive entries per
// turn: one 4-byte load per lane, one ballot, one 8-byte store (partial at the end).
// Vote: out[k] = scale * sign(sum_m (2 b_m[k] - 1)), a tie counting as +1.  A thread
// takes 32 consecutive entries (one 32-bit word of every worker's buffer); the counts are
// kept bit-sliced (see sign_vote_kernel), and a wave's 2048 results are redistributed
// across its lanes so that every store instruction writes one contiguous run.  Both are
// HBM-bound streams.

#include <type_traits>

#include "device_common.h"
#include "himuon_internal.h"

namespace himuon {
namespace {

using namespace dev;

constexpr int SIGN_THREADS = 256;

// UNROLL turns of 64 entries per wave per loop iteration: their loads are all issued
// before the first ballot, so each wave keeps UNROLL loads in flight.
constexpr int PACK_UNROLL = 8;

template <bool CONTIG>
__global__ __launch_bounds__(SIGN_THREADS) void sign_pack_kernel(const float *__restrict__ o, int64_t cols, int64_t ld,
                                                                 int64_t n, unsigned char *__restrict__ bits) {
  const int lane = threadIdx.x & 63;
  const int64_t turns = (n + 63) / 64;
  const int64_t waves = (int64_t)gridDim.x * (SIGN_THREADS / 64);
  for (int64_t c0 = ((int64_t)blockIdx.x * (SIGN_THREADS / 64) + (threadIdx.x >> 6)) * PACK_UNROLL; c0 < turns;
       c0 += waves * PACK_UNROLL) {
    float v[PACK_UNROLL];
#pragma unroll
    for (int u = 0; u < PACK_UNROLL; ++u) {
      const int64_t k = (c0 + u) * 64 + lane;
      v[u] = -1.f;
      if (k < n) v[u] = gmem(o)[CONTIG ? k : (k / cols) * ld + k % cols];
    }
#pragma unroll
    for (int u = 0; u < PACK_UNROLL; ++u) {
      const int64_t c = c0 + u;
      if (c >= turns) break;   // wave-uniform
      const unsigned long long m = __ballot(v[u] >= 0.f);
      const int64_t rem = n - c * 64;   // entries of this turn that exist
      if (rem >= 64) {
        if (lane == 0) *gmem(reinterpret_cast<unsigned long long *>(bits + c * 8)) = m;
      } else if (lane < (rem + 7) / 8) {
        gmem(bits)[c * 8 + lane] = (unsigned char)(m >> (8 * lane));
      }
    }
  }
}

// Bit i of an 8-bit value moved to bit 4 i of the result.
__device__ __forceinline__ unsigned int spread4(unsigned int x) {
  x &= 0xffu;
  x = (x | (x << 12)) & 0x000f000fu;
  x = (x | (x << 6)) & 0x03030303u;
  x = (x | (x << 3)) & 0x11111111u;
  return x;
}

// Contiguous 16-byte aligned input: a wave takes 256 consecutive entries per turn, four
// per lane in one 16-byte load.  Ballot e collects element e of every lane (bit l = entry
// 4 l + e); output word k (entries 32 k .. 32 k + 31, lanes 8 k .. 8 k + 7) interleaves
// byte k of the four ballots, and lanes 0..7 store the turn's eight words.
__global__ __launch_bounds__(SIGN_THREADS) void sign_pack4_kernel(const float *__restrict__ o, int64_t n,
                                                                  unsigned char *__restrict__ bits) {
  const int lane = threadIdx.x & 63;
  const int64_t turns = (n + 255) / 256;
  const int64_t nbytes = (n + 7) / 8;
  const int64_t waves = (int64_t)gridDim.x * (SIGN_THREADS / 64);
  for (int64_t c0 = ((int64_t)blockIdx.x * (SIGN_THREADS / 64) + (threadIdx.x >> 6)) * PACK_UNROLL; c0 < turns;
       c0 += waves * PACK_UNROLL) {
    f32x4 v[PACK_UNROLL];
#pragma unroll
    for (int u = 0; u < PACK_UNROLL; ++u) {
      const int64_t k = (c0 + u) * 256 + 4 * lane;
      if (k + 4 <= n) {
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const GLOBAL_AS f32x4 *>(gmem(o + k)));
      } else {
        v[u] = f32x4{-1.f, -1.f, -1.f, -1.f};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (k + e < n) v[u][e] = gmem(o)[k + e];
      }
    }
#pragma unroll
    for (int u = 0; u < PACK_UNROLL; ++u) {
      const int64_t c = c0 + u;
      if (c >= turns) break;   // wave-uniform
      unsigned int word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned long long m = __ballot(v[u][e] >= 0.f);
        word |= spread4((unsigned int)(m >> (8 * (lane & 7)))) << e;
      }
      const int64_t b0 = c * 32 + 4 * lane;   // first output byte of lane < 8
      if (lane < 8) {
        if (b0 + 4 <= nbytes) {
          *gmem(reinterpret_cast<unsigned int *>(bits + b0)) = word;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (b0 + j < nbytes) gmem(bits)[b0 + j] = (unsigned char)(word >> (8 * j));
        }
      }
    }
  }
}

// The vote counts bit-sliced: plane b of a 32-bit word holds bit b of the 32 counts, a
// worker's word is added with a ripple of half adders over NP planes (NP = 4 holds up to
// 15 workers, 8 up to 255), and count >= ceil(workers / 2) is decided plane by plane
// from the most significant one.  Workers are read in groups of 8 whose loads are all
// issued before any is added.
template <typename OUT, int NP>
__global__ __launch_bounds__(SIGN_THREADS) void sign_vote_kernel(const unsigned char *__restrict__ bits, int workers,
                                                                 int64_t stride, int64_t n, OUT *__restrict__ out,
                                                                 float scale) {
  const int64_t words = (n + 31) / 32;
  const int thr = (workers + 1) / 2;   // 2 count >= workers  <=>  count >= thr
  for (int64_t w = (int64_t)blockIdx.x * SIGN_THREADS + threadIdx.x; w < words;
       w += (int64_t)gridDim.x * SIGN_THREADS) {
    const int64_t nb = n - w * 32 < 32 ? (n - w * 32 + 7) / 8 : 4;   // bytes of this word present
    unsigned int plane[NP];
#pragma unroll
    for (int b = 0; b < NP; ++b) plane[b] = 0;
    for (int m0 = 0; m0 < workers; m0 += 8) {
      unsigned int xs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        xs[u] = 0;
        const int m = m0 + u;
        if (m < workers) {
          const unsigned char *src = bits + (int64_t)m * stride + w * 4;
          if (nb == 4) {
            xs[u] = *gmem(reinterpret_cast<const unsigned int *>(src));
          } else {
            for (int b = 0; b < nb; ++b) xs[u] |= (unsigned int)gmem(src)[b] << (8 * b);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        unsigned int carry = xs[u];
#pragma unroll
        for (int b = 0; b < NP; ++b) {
          const unsigned int t = plane[b] & carry;
          plane[b] ^= carry;
          carry = t;
        }
      }
    }
    unsigned int gt = 0, eq = 0xffffffffu;
#pragma unroll
    for (int b = NP - 1; b >= 0; --b) {
      if ((thr >> b) & 1) {
        eq &= plane[b];
      } else {
        gt |= eq & plane[b];
        eq &= ~plane[b];
      }
    }
    const unsigned int ge = gt | eq;   // bit j: entry j wins +1
    // Whole waves (64 full words, 2048 entries) store coalesced: store instruction q of
    // lane l covers entries q * 64 * EPS + l * EPS .. + EPS - 1 of the wave (EPS = 16 /
    // sizeof(OUT) per 16-byte store), whose bits sit in the word of lane (q * 64 * EPS +
    // l * EPS) / 32, fetched with ds_bpermute.  The condition is wave-uniform.
    const int64_t wave_w0 = w - (threadIdx.x & 63);
    if ((wave_w0 + 64) * 32 <= n && ((reinterpret_cast<uintptr_t>(out) & 15) == 0)) {
      constexpr int EPS = 16 / (int)sizeof(OUT);   // entries per 16-byte store: 8 or 4
      constexpr int NQ = 2048 / (64 * EPS);        // stores per lane: 4 or 8
      const int l = threadIdx.x & 63;
      OUT *base = out + wave_w0 * 32;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int e0 = q * 64 * EPS + l * EPS;     // first entry (within the wave) of this store
        const unsigned int word = (unsigned int)__builtin_amdgcn_ds_bpermute((e0 >> 5) * 4, (int)ge);
        const unsigned int bits = word >> (e0 & 31);
        if constexpr (sizeof(OUT) == 4) {
          f32x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = ((bits >> j) & 1u) ? scale : -scale;
          *reinterpret_cast<GLOBAL_AS f32x4 *>(gmem(reinterpret_cast<float *>(base + e0))) = v;
        } else {
          float v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = ((bits >> j) & 1u) ? scale : -scale;
          *reinterpret_cast<GLOBAL_AS u32x4 *>(gmem(reinterpret_cast<__bf16 *>(base + e0))) =
              u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7])};
        }
      }
      continue;
    }
    const int64_t k0 = w * 32;
    const int cnt_n = n - k0 < 32 ? (int)(n - k0) : 32;
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = ((ge >> j) & 1u) ? scale : -scale;
    if (cnt_n == 32 && ((reinterpret_cast<uintptr_t>(out) & 15) == 0)) {
      if constexpr (sizeof(OUT) == 4) {
        GLOBAL_AS f32x4 *d = reinterpret_cast<GLOBAL_AS f32x4 *>(gmem(reinterpret_cast<float *>(out) + k0));
#pragma unroll
        for (int q = 0; q < 8; ++q) d[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
      } else {
        GLOBAL_AS u32x4 *d = reinterpret_cast<GLOBAL_AS u32x4 *>(gmem(reinterpret_cast<__bf16 *>(out) + k0));
#pragma unroll
        for (int q = 0; q < 4; ++q)
          d[q] = u32x4{pack_bf16x2(v[8 * q], v[8 * q + 1]), pack_bf16x2(v[8 * q + 2], v[8 * q + 3]),
                       pack_bf16x2(v[8 * q + 4], v[8 * q + 5]), pack_bf16x2(v[8 * q + 6], v[8 * q + 7])};
      }
    } else {
      for (int j = 0; j < cnt_n; ++j) gmem(out)[k0 + j] = (OUT)v[j];
    }
  }
}

int grid_for(int64_t items, int64_t per_block) {
  const int64_t g = (items + per_block - 1) / per_block;
  return (int)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

}  // namespace

hipError_t launch_sign_pack(const float *o, int64_t rows, int64_t cols, int64_t ld, unsigned char *bits,
                            hipStream_t stream) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  if (ld == cols && (reinterpret_cast<uintptr_t>(o) & 15) == 0) {
    const int grid4 = grid_for((n + 255) / 256, (SIGN_THREADS / 64) * PACK_UNROLL);
    hipLaunchKernelGGL(sign_pack4_kernel, dim3(grid4), dim3(SIGN_THREADS), 0, stream, o, n, bits);
    return hipGetLastError();
  }
  const int grid = grid_for((n + 63) / 64, (SIGN_THREADS / 64) * PACK_UNROLL);
  if (ld == cols) {
    hipLaunchKernelGGL(sign_pack_kernel<true>, dim3(grid), dim3(SIGN_THREADS), 0, stream, o, cols, ld, n, bits);
  } else {
    hipLaunchKernelGGL(sign_pack_kernel<false>, dim3(grid), dim3(SIGN_THREADS), 0, stream, o, cols, ld, n, bits);
  }
  return hipGetLastError();
}

hipError_t launch_sign_vote(const unsigned char *bits, int workers, int64_t stride, int64_t n, bool out_bf16,
                            void *out, float scale, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int grid = grid_for((n + 31) / 32, SIGN_THREADS);
  auto go = [&](auto np) {
    constexpr int NP = decltype(np)::value;
    if (out_bf16) {
      hipLaunchKernelGGL((sign_vote_kernel<__bf16, NP>), dim3(grid), dim3(SIGN_THREADS), 0, stream, bits, workers,
                         stride, n, reinterpret_cast<__bf16 *>(out), scale);
    } else {
      hipLaunchKernelGGL((sign_vote_kernel<float, NP>), dim3(grid), dim3(SIGN_THREADS), 0, stream, bits, workers,
                         stride, n, reinterpret_cast<float *>(out), scale);
    }
  };
  if (workers <= 15) {
    go(std::integral_constant<int, 4>{});
  } else {
    go(std::integral_constant<int, 8>{});
  }
  return hipGetLastError();
}

}  // namespace himuon
