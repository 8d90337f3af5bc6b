// select.h -- exact selection of the best records by radix select (one wave).
//
// A record is the 64-bit key (monotone score code << 32) | (~key index), so
// ordering records descending orders by score descending, then key index
// ascending.  Records are distinct (one per key), so "the `need` largest
// records" is a unique set.
//
// A selection is (prefix, mask): the kept records are those r with
// (r & mask) >= prefix.  Digits come from the top, 8 bits at a time; it
// stops as soon as the digit bin holding the boundary is taken whole
// (exact), or -- for a mid-scan cut of a candidate buffer -- as soon as the
// kept count is small enough.  `prefix` is always a valid running
// threshold: every record below it is beaten by at least `need` kept
// records.  Passes read the buffer 8 records per lane at a time so that
// many loads are in flight.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

struct SelectResult {
  uint64_t prefix;
  uint64_t mask;
  uint32_t kept;  // number of records with (r & mask) >= prefix
};

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

// Boundary bin of an nb-bin histogram: the highest bin b with
// count(bins >= b) >= remaining.  Returns b, the count strictly above it and
// its own count, in every lane.
__device__ __forceinline__ void find_boundary(const uint32_t* hist, uint32_t nb, uint32_t remaining, int lane,
                                              uint32_t& bin, uint32_t& above, uint32_t& count) {
  const uint32_t bpl = nb / 64;
  uint32_t local = 0;
  for (uint32_t j = 0; j < bpl; ++j) local += hist[lane * bpl + j];
  const uint32_t sfx = wave_suffix_excl(local, lane);
  const bool mine = sfx < remaining && remaining <= sfx + local;
  const uint64_t bal = __ballot(mine);
  const int src = __builtin_ctzll(bal);
  uint32_t b = 0, a = 0, c = 0;
  if (lane == src) {
    uint32_t acc = sfx;
    for (int j = (int)bpl - 1; j >= 0; --j) {
      const uint32_t h = hist[lane * bpl + j];
      if (acc + h >= remaining) {
        b = lane * bpl + j;
        a = acc;
        c = h;
        break;
      }
      acc += h;
    }
  }
  bin = __shfl(b, src, 64);
  above = __shfl(a, src, 64);
  count = __shfl(c, src, 64);
}

// Histogram of digit (S, nb) over the records of buf[0, cnt) that match
// (prefix, mask).  hist must be cleared by the caller.
__device__ __forceinline__ void hist_pass(const uint64_t* buf, int cnt, uint64_t prefix, uint64_t mask, int S,
                                          uint32_t nb, uint32_t* hist, int lane) {
  for (int i0 = 0; i0 < cnt; i0 += 512) {
    uint64_t r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j + lane;
      r[j] = i < cnt ? buf[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j + lane;
      if (i < cnt && (r[j] & mask) == prefix) atomicAdd(&hist[(uint32_t)(r[j] >> S) & (nb - 1)], 1u);
    }
  }
}

// Select the `need` best of the cnt records in buf (1 <= need <= cnt): up
// to eight passes of 8-bit digits over a 256-bin histogram, each pass
// reading the buffer.  exact = false stops once kept <= goal.
static __device__ __noinline__ SelectResult select_records_d8(const uint64_t* buf, int cnt, uint32_t need,
                                                              uint32_t* hist, bool exact, uint32_t goal, int lane) {
  uint64_t prefix = 0, mask = 0;
  uint32_t remaining = need, kept = (uint32_t)cnt;
  for (int pass = 0; pass < 8; ++pass) {
    const int S = 56 - 8 * pass;
    for (uint32_t i = lane; i < 256; i += 64) hist[i] = 0;
    hist_pass(buf, cnt, prefix, mask, S, 256, hist, lane);
    uint32_t bin, above, count;
    find_boundary(hist, 256, remaining, lane, bin, above, count);
    prefix |= (uint64_t)bin << S;
    mask |= (uint64_t)0xFF << S;
    remaining -= above;
    kept = need - remaining + count;
    if (count == remaining) break;  // boundary bin taken whole: exact
    if (!exact && kept <= goal) break;
  }
  return {prefix, mask, kept};
}

// In place: keep records with (r & mask) >= prefix, in their order.
// Returns the kept count.
static __device__ __noinline__ int compact_records_d8(uint64_t* buf, int cnt, SelectResult sel, int lane) {
  int base = 0;
  for (int i0 = 0; i0 < cnt; i0 += 512) {
    uint64_t r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j + lane;
      r[j] = i < cnt ? buf[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j + lane;
      const bool keep = i < cnt && (r[j] & sel.mask) >= sel.prefix;
      const uint64_t bal = __ballot(keep);
      const uint32_t before =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (keep) buf[base + before] = r[j];
      base += __popcll(bal);
    }
  }
  return base;
}

// Smallest of the cnt records in buf (all lanes get it; ~0 if cnt == 0).
static __device__ __noinline__ uint64_t min_record(const uint64_t* buf, int cnt, int lane) {
  uint64_t mn = ~0ull;
  for (int i = lane; i < cnt; i += 64) mn = buf[i] < mn ? buf[i] : mn;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const uint64_t o = __shfl_xor(mn, d, 64);
    mn = o < mn ? o : mn;
  }
  return mn;
}

}  // namespace dsa
