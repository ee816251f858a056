// kernels_common.h -- launch arguments and small device helpers shared by the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "group_addr.h"

namespace ma {

// One launch runs softmax attention independently inside every token group
// of every (batch, head): out[g] = softmax(s q[g] k[g]^T) vals[g].
struct AttnLaunch {
  const void *q;
  const void *k;
  const void *vals;   // V (stage R, dense) or Y (stage L)
  void *out;
  int64_t head_elems; // N * head_dim: distance between consecutive (batch, head) slices
  GroupAddr ga;
  int32_t n_qtiles;   // query tiles per group, or per query span (sized for the largest)
  int32_t q_tile;     // queries per query tile (streaming bf16 kernel)
  // Query ranges of the streaming bf16 kernel (other kernels take 0, 0, 1):
  // members below q_first are keys only; with q_span > 0 the queries from
  // q_first on are cut into n_spans spans of q_span members, and span s
  // attends to members [0, q_first + (s+1) q_span) only (chunk-causal).
  int32_t q_first;
  int32_t q_span;
  int32_t n_spans;
  // span_waves > 0 (several spans): spans are cut into wave items of 32
  // queries (span_waves per span, last_waves in the last one), ordered by
  // span from the last to the first, and workgroup qt of a group runs items
  // qt*NW .. qt*NW+NW-1, one per wave; n_qtiles counts those workgroups.
  int32_t span_waves;
  int32_t last_waves;
  int32_t n_bh;       // batch * heads
  float scale;        // 1/sqrt(head_dim)
  float scale_log2;   // scale * log2(e): softmax evaluated with exp2
};

}  // namespace ma
