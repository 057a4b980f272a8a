// Internal launch functions behind the C ABI (host side), and the optional
// per-kernel event recorder used by ulysses_profile_*.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uly {

struct AttnArgs;

hipError_t permute_launch(bool pack, const void* src, void* dst, int P, int B, int S, int H, int D,
                          int elem_bytes, hipStream_t st);
hipError_t segments_launch(const void* pos, int pos_bytes, int P, int B, int S, int32_t* cu,
                           int32_t* n_seqs, int32_t* max_len, hipStream_t st);
hipError_t attn_fwd_launch(const AttnArgs& a, int D, hipStream_t st);
hipError_t attn_bwd_launch(const AttnArgs& a, int D, hipStream_t st);
void dkdv_launch(const AttnArgs& a, int D, hipStream_t st);  // part of attn_bwd_launch

// When profiling is on, prof_mark(name, st) records a HIP event on `st`
// before a kernel launch and prof_mark(nullptr, st) after it.
void prof_mark(const char* name, hipStream_t st);

struct ProfScope {
  hipStream_t st;
  ProfScope(const char* name, hipStream_t s) : st(s) { prof_mark(name, s); }
  ~ProfScope() { prof_mark(nullptr, st); }
};

}  // namespace uly
