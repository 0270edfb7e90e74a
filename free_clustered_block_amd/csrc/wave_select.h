// One-wave selection shared by the split and the routing kernels: of the n
// members (n <= kWaveSelMax, 16 keys per lane) the t smallest in strict
// (key, position) order are taken. Radix select over 8-bit digits from the
// highest bit in which the keys differ, with a per-wave LDS histogram and
// wave-wide ballots, no workgroup barriers; then every member is visited in
// position order with whether it is taken and its rank among the taken
// (emit(i, taken, rank)).
#pragma once

#include "common.h"

namespace ca {

constexpr int kWaveSelMax = 1024;

CA_DEV void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// l: lane; key_at(i): key of member i (i < n); hw: the wave's 256-int histogram
template <typename KeyAt, typename Emit>
CA_DEV void wave_select(int l, int n, int t, KeyAt key_at, int* hw, Emit emit) {
  constexpr int KPL = kWaveSelMax / 64;   // keys per lane
  uint32_t k[KPL];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int q = 0; q < KPL; ++q) {
    const int i = l + 64 * q;
    k[q] = i < n ? key_at(i) : 0u;
    if (i < n) { kmin = min(kmin, k[q]); kmax = max(kmax, k[q]); }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, d, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d, 64));
  }
  const uint32_t diff = kmin ^ kmax;
  const int hb = diff ? 31 - __builtin_clz(diff) : -1;
  uint32_t prefix = hb < 0 ? kmin : (hb == 31 ? 0u : kmin & (0xFFFFFFFFu << (hb + 1)));
  int want = t;
  for (int hi = hb; hi >= 0;) {
    const int lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (2u << (hi - lo)) - 1u;
    const uint32_t hmask = hi == 31 ? 0u : (0xFFFFFFFFu << (hi + 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) hw[4 * l + j] = 0;
    wave_sync();
#pragma unroll
    for (int q = 0; q < KPL; ++q)
      if (l + 64 * q < n && (k[q] & hmask) == (prefix & hmask)) atomicAdd(&hw[(k[q] >> lo) & dmask], 1);
    wave_sync();
    int v[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { v[j] = hw[4 * l + j]; s += v[j]; }
    int inc = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(inc, d, 64);
      if (l >= d) inc += y;
    }
    int before = inc - s, bsel = 0, bbefore = 0;
    bool mine = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (before < want && want <= before + v[j]) { mine = true; bsel = 4 * l + j; bbefore = before; }
      before += v[j];
    }
    const uint64_t owner = __ballot(mine);
    const int src = owner ? __builtin_ctzll(owner) : 0;   // one lane owns rank `want`
    bsel = __shfl(bsel, src, 64);
    bbefore = __shfl(bbefore, src, 64);
    prefix |= (uint32_t)bsel << lo;
    want -= bbefore;
    hi = lo - 1;
    wave_sync();   // every lane has read the histogram before it is cleared again
  }
  const uint32_t kstar = prefix;
  const int eq_take = want;
  int erun = 0, lrun = 0;
#pragma unroll
  for (int q = 0; q < KPL; ++q) {
    const int i = l + 64 * q;
    if (64 * q >= n) break;   // uniform
    const bool valid = i < n;
    const bool less = valid && k[q] < kstar;
    const bool eq = valid && k[q] == kstar;
    uint64_t bal_e, bal_l;
    const int eqpre = lane_prefix(eq, &bal_e);
    const bool left = less || (eq && erun + eqpre < eq_take);
    const int lpre = lane_prefix(left, &bal_l);
    const int lrank = lrun + lpre;
    if (valid) emit(i, left, lrank);
    erun += __popcll(bal_e);
    lrun += __popcll(bal_l);
  }
}

}  // namespace ca
