// M tile of the grouped GEMMs by mean token-expert pairs per expert, written by
// fp8_block_scaled_grouped_amd/tuning/make_tables.py from block_m_sweep.jsonl.
// An entry serves T * topk / E <= ppe_max (the first such entry); above the last,
// the last entry's tile.  Whole-layer milliseconds per swept tile in comments.
#pragma once

namespace moe355 {

struct BlockMTuned {
  double ppe_max;
  int block_m;
};

static const BlockMTuned kBlockMTuned[] = {
    {2, 16},  // 16:1.009 32:1.021 64:1.036 128:1.053 256:1.308
    {4, 32},  // 16:1.265 32:1.255 64:1.274 128:1.295 256:1.607
    {16, 64},  // 16:1.862 32:1.651 64:1.620 128:1.625 256:2.072
    {256, 128},  // 16:13.516 32:8.564 64:5.912 128:4.756 256:5.504
};

}  // namespace moe355
