// Shared device helpers for the libsfx kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sfx {

constexpr int kWave = 64;
constexpr int kBlock = 256;          // threads per workgroup for the streaming kernels
constexpr int kWavesPerBlock = kBlock / kWave;

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_Q4 = 3 };

// Storage traits.  `vec` = elements in one 16-byte load.
struct TF32 { static constexpr int bytes = 4; static constexpr int vec = 4; };
struct TF16 { static constexpr int bytes = 2; static constexpr int vec = 8; };
struct TBF16 { static constexpr int bytes = 2; static constexpr int vec = 8; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Exact conversion of one 32-bit word holding storage elements to floats.
__device__ __forceinline__ void unpack_word(TF32, uint32_t w, float* o) { o[0] = __uint_as_float(w); }
__device__ __forceinline__ void unpack_word(TF16, uint32_t w, float* o) {
  half2_t h = __builtin_bit_cast(half2_t, w);
  o[0] = (float)h.x;
  o[1] = (float)h.y;
}
__device__ __forceinline__ void unpack_word(TBF16, uint32_t w, float* o) {
  o[0] = __uint_as_float(w << 16);
  o[1] = __uint_as_float(w & 0xFFFF0000u);
}

template <class T>
struct PerWord { static constexpr int n = 4 / T::bytes; };

// `NW` 32-bit words -> NW * (4 / bytes) floats.
template <class T, int NW>
__device__ __forceinline__ void unpack(const uint32_t* w, float* o) {
#pragma unroll
  for (int i = 0; i < NW; ++i) unpack_word(T{}, w[i], o + i * PerWord<T>::n);
}

// A load of N bytes (N = 4, 8 or 16) as one vector instruction.
template <int N>
struct alignas(N) Raw { uint32_t w[N / 4]; };

template <int N>
__device__ __forceinline__ Raw<N> load_raw(const void* p) { return *reinterpret_cast<const Raw<N>*>(p); }


// Sum each of V values (V a power of two, V <= 64) over the 64 lanes of a wave,
// halving the values held per lane at every exchange (about V + 6 shuffles instead
// of 6 V).  On return v[0] of lane L holds the total of value index
// L >> (6 - log2 V).  The pattern is fixed, so results are reproducible.
// Lane index behind an opaque copy: lane masks derived from threadIdx.x directly
// are loop-invariant, get hoisted out of long loops and pin scalar registers.
__device__ __forceinline__ int opaque_lane() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t & (kWave - 1);
}

// Value of lane L ^ O (O = 8, 4, 2, 1) by DPP within rows of 16 lanes: VALU
// operations, no LDS crossbar round trip.  Xor 4 takes row_shr:4 on lanes with bit
// 2 set and row_shl:4 on the others.
template <int O>
__device__ __forceinline__ float lane_xor_dpp(float x, int lane) {
  const int xi = __float_as_int(x);
  if constexpr (O == 8) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0x128, 0xf, 0xf, false));   // row_ror:8
  } else if constexpr (O == 4) {
    const int from_below = __builtin_amdgcn_update_dpp(0, xi, 0x114, 0xf, 0xf, false);  // row_shr:4
    const int from_above = __builtin_amdgcn_update_dpp(0, xi, 0x104, 0xf, 0xf, false);  // row_shl:4
    return __int_as_float((lane & 4) ? from_below : from_above);
  } else if constexpr (O == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0x4e, 0xf, 0xf, false));    // quad_perm 2,3,0,1
  } else {
    static_assert(O == 1, "lane_xor_dpp: O in 1, 2, 4, 8");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, xi, 0xb1, 0xf, 0xf, false));    // quad_perm 1,0,3,2
  }
}
// 32-bit value of lane L ^ O, any O in 32, 16, 8, 4, 2, 1 (lane swaps for 32 and
// 16, DPP below): VALU operations only.
template <int O>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t x, int lane) {
  if constexpr (O == 32 || O == 16) {
    const auto r = O == 32 ? __builtin_amdgcn_permlane32_swap(x, x, false, false)
                           : __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & O) ? r[0] : r[1];
  } else {
    return __float_as_uint(lane_xor_dpp<O>(__uint_as_float(x), lane));
  }
}
// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within rows of 16,
// then lane 15 added to rows 1 and 3 and lane 31 to rows 2 and 3 (DPP row
// broadcasts).
__device__ __forceinline__ uint32_t wave_inclusive_scan_u32(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return (uint32_t)v;
}
// Butterfly sum over the 64 lanes of a wave (lane L with L ^ 32, then 16, ..., 1);
// every lane gets the total.  The order of additions is fixed, so the result is
// reproducible.
__device__ __forceinline__ float wave_sum(float v) {
  int lane = threadIdx.x;
  asm volatile("" : "+v"(lane));
  lane &= kWave - 1;
  v += __uint_as_float(lane_xor_u32<32>(__float_as_uint(v), lane));
  v += __uint_as_float(lane_xor_u32<16>(__float_as_uint(v), lane));
  v += __uint_as_float(lane_xor_u32<8>(__float_as_uint(v), lane));
  v += __uint_as_float(lane_xor_u32<4>(__float_as_uint(v), lane));
  v += __uint_as_float(lane_xor_u32<2>(__float_as_uint(v), lane));
  v += __uint_as_float(lane_xor_u32<1>(__float_as_uint(v), lane));
  return v;
}
// Sum over the 64 lanes, every lane ends with it.
__device__ __forceinline__ int wave_sum_i32(int v, int lane) {
  v += (int)lane_xor_u32<32>((uint32_t)v, lane);
  v += (int)lane_xor_u32<16>((uint32_t)v, lane);
  v += (int)lane_xor_u32<8>((uint32_t)v, lane);
  v += (int)lane_xor_u32<4>((uint32_t)v, lane);
  v += (int)lane_xor_u32<2>((uint32_t)v, lane);
  v += (int)lane_xor_u32<1>((uint32_t)v, lane);
  return v;
}

// a (lanes kept by the lower half of each 2 O block) + b (kept by the upper
// half) exchanged across lane bit O = 32 or 16 with the gfx950 lane-swap
// instructions: returns, in lane L, the sum of L's and (L ^ O)'s values of the
// element L keeps (a below, b above).
template <int O>
__device__ __forceinline__ float swap_add(float a, float b) {
  const auto r = O == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                         : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Halving reduction: at lane bit O the lanes with the bit clear keep the first
// half of the values, the others the second half, each adding its partner's.
// The pairing (L with L ^ O) and the order of every addition are those of a
// plain exchange by lane xor.
template <int V, int O, int M = 1>
struct WaveReduceStep {
  __device__ __forceinline__ static void run(float* v, int lane) {
    constexpr int half = V / 2;
    if constexpr (O >= 16) {
#pragma unroll
      for (int i = 0; i < half; ++i) v[i] = swap_add<O>(v[i], v[i + half]);
    } else {
      const bool up = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float send = up ? v[i] : v[i + half];
        const float keep = up ? v[i + half] : v[i];
        v[i] = keep + lane_xor_dpp<O>(send, lane);
      }
    }
    WaveReduceStep<half, O / 2, M>::run(v, lane);
  }
};
template <int O, int M>
struct WaveReduceStep<1, O, M> {
  __device__ __forceinline__ static void run(float* v, int lane) {
    if constexpr (O >= M) {
      if constexpr (O >= 16) v[0] = swap_add<O>(v[0], v[0]);
      else v[0] += lane_xor_dpp<O>(v[0], lane);
      WaveReduceStep<1, O / 2, M>::run(v, lane);
    }
  }
};
template <int M>
struct WaveReduceStep<1, 0, M> {
  __device__ __forceinline__ static void run(float*, int) {}
};
template <int V>
__device__ __forceinline__ float wave_reduce_multi(float (&v)[V]) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
  WaveReduceStep<V, 32>::run(v, opaque_lane());
  return v[0];
}
// As wave_reduce_multi, but lanes are only summed across lane bits >= log2 M:
// lane L ends with value index L >> (6 - log2 V) of lane group L mod M, and lanes
// with (L mod 64/V) < M hold distinct (index, group) pairs.
template <int V, int M>
__device__ __forceinline__ float wave_reduce_multi_groups(float (&v)[V]) {
  static_assert(V >= 1 && V * M <= 64 && (V & (V - 1)) == 0 && (M & (M - 1)) == 0, "bad V / M");
  WaveReduceStep<V, 32, M>::run(v, opaque_lane());
  return v[0];
}
__host__ __device__ constexpr int ilog2c(int v) { return v <= 1 ? 0 : 1 + ilog2c(v / 2); }

// Cross-workgroup hand-off without a device-wide cache write-back.  A producer
// writes the data it hands over with agent-scope atomic stores (written through to
// the coherence point), waits for them to complete and then bumps a ticket with a
// relaxed agent-scope atomic.  The consumer that sees the final ticket invalidates
// its caches once (agent acquire) and reads the data with ordinary loads.  This
// avoids an agent release fence in every producer, whose L2 write-back is
// serialised across the device.
__device__ __forceinline__ void store_through(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_through(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_through2(float* p, float a, float b) {  // p 8-byte aligned
  const unsigned long long v = ((unsigned long long)__float_as_uint(b) << 32) | __float_as_uint(a);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this thread's outstanding memory operations have completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }
// Ticket: returns the previous value (relaxed, agent scope).
__device__ __forceinline__ uint32_t take_ticket(uint32_t* t) {
  return __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Consumer side: drop stale cache lines before reading handed-over data.
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Token-count classes that kernels are instantiated for.
__host__ __device__ constexpr int nb_class(int B) {
  return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : B <= 16 ? 16 : B <= 32 ? 32 : 64;
}

}  // namespace sfx
