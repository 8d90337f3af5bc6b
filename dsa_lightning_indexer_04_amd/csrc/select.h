// select.h -- exact selection of the best records by radix select.
//
// A record is the 64-bit key (monotone score code << 32) | (~key index), so
// ordering records descending orders by score descending, then key index
// ascending.  Records are distinct (one per key), so "the `need` largest
// records" is a unique set.
//
// The select finds (prefix, mask): the `need` largest records are exactly
// those r with (r & mask) >= prefix.  Digits are taken from the top, 11/11/10
// bits of the score code and then of the key part; it stops as soon as the
// digit bin holding the boundary is taken whole.  `prefix` is also a valid
// running threshold: every record below it is beaten by at least `need`
// records.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

struct SelectResult {
  uint64_t prefix;
  uint64_t mask;
};

__device__ __forceinline__ int digit_shift(int pass) {
  const int s[6] = {53, 42, 32, 21, 10, 0};
  return s[pass];
}
__device__ __forceinline__ int digit_width(int pass) { return (pass == 2 || pass == 5) ? 10 : 11; }

// Wave-wide exclusive suffix sum of `x` over lanes above this one.
__device__ __forceinline__ uint32_t wave_suffix_excl(uint32_t x, int lane) {
  uint32_t incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t y = __shfl_down(incl, d, 64);
    if (lane + d < 64) incl += y;
  }
  return incl - x;
}

// One wave selects among `cnt` records at `buf` (global memory).  hist is a
// 2048-entry LDS scratch private to the wave.  Requires 1 <= need <= cnt.
__device__ __noinline__ SelectResult wave_radix_select(const uint64_t* buf, int cnt, int need, uint32_t* hist,
                                                       int lane) {
  uint64_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)need;
  for (int pass = 0; pass < 6; ++pass) {
    const int S = digit_shift(pass), W = digit_width(pass);
    const uint32_t nb = 1u << W, bpl = nb / 64;
    for (uint32_t i = lane; i < nb; i += 64) hist[i] = 0;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    for (int i = lane; i < cnt; i += 64) {
      uint64_t r = buf[i];
      if ((r & mask) == prefix) atomicAdd(&hist[(uint32_t)(r >> S) & (nb - 1)], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    uint32_t local = 0;
    for (uint32_t j = 0; j < bpl; ++j) local += hist[lane * bpl + j];
    uint32_t above = wave_suffix_excl(local, lane);
    bool mine = above < remaining && remaining <= above + local;
    uint64_t bal = __ballot(mine);
    int src = __builtin_ctzll(bal);
    uint32_t dsel = 0, dabove = 0, dcount = 0;
    if (lane == src) {
      uint32_t acc = above;
      for (int j = (int)bpl - 1; j >= 0; --j) {
        uint32_t h = hist[lane * bpl + j];
        if (acc + h >= remaining) {
          dsel = lane * bpl + j;
          dabove = acc;
          dcount = h;
          break;
        }
        acc += h;
      }
    }
    dsel = __shfl(dsel, src, 64);
    dabove = __shfl(dabove, src, 64);
    dcount = __shfl(dcount, src, 64);
    prefix |= (uint64_t)dsel << S;
    mask |= (uint64_t)(nb - 1) << S;
    remaining -= dabove;
    __builtin_amdgcn_wave_barrier();
    if (dcount == remaining) break;
  }
  return {prefix, mask};
}

}  // namespace dsa
