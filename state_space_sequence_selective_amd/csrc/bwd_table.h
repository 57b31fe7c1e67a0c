// Configurations of the backward kernel per (d_state, checkpoint interval L):
//   X(DS, L, SPL, SUB, PD, W, PDF, WF)
// SPL states per thread, SUB steps per sub-tile, then the operand look-ahead
// and the waves per SIMD the register allocation targets, for the scan entry
// (PD, W) and for the fused entry (PDF, WF).  A thread keeps h_t and dA_t of
// its SPL states for all L steps of a tile in registers (2 * SPL * L of
// them); a workgroup must be whole waves.  Three waves per SIMD hide the LDS
// and barrier waits best (measured: T=8192 backward 2.04 -> 1.81 ms) where
// the registers allow it without spilling (168 or fewer: the look-ahead is
// shortened to fit).  The launcher (scan_bwd.h) and the segment planner
// (abi.hip) both read this one list.
#pragma once

#define MSCAN_BWD_CONFIGS(X)                                     \
  X(4, 16, 1, 4, 4, 3, 4, 2) X(4, 32, 1, 4, 1, 2, 1, 2)          \
  X(8, 16, 2, 4, 4, 2, 4, 2) X(8, 32, 1, 8, 4, 2, 4, 2)          \
  X(16, 16, 2, 8, 1, 3, 1, 3) X(16, 32, 1, 8, 4, 2, 4, 2)        \
  X(32, 16, 2, 8, 4, 2, 4, 2) X(64, 16, 4, 4, 4, 2, 4, 2)

namespace mscan {

// states per thread of the backward kernel of this configuration (0: none)
inline int bwd_states_per_thread(int ds, int L) {
#define MSCAN_S(DS_, L_, SPL_, SUB_, PD_, W_, PDF_, WF_) \
  if (ds == DS_ && L == L_) return SPL_;
  MSCAN_BWD_CONFIGS(MSCAN_S)
#undef MSCAN_S
  return 0;
}

// waves per SIMD the backward kernel of this configuration is built for
// (0: no such configuration)
inline int bwd_waves_per_simd(int ds, int L, bool fused) {
#define MSCAN_W(DS_, L_, SPL_, SUB_, PD_, W_, PDF_, WF_) \
  if (ds == DS_ && L == L_) return fused ? WF_ : W_;
  MSCAN_BWD_CONFIGS(MSCAN_W)
#undef MSCAN_W
  return 0;
}

}  // namespace mscan
