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
    {2, 16},  // 16:1.019 32:1.029 64:1.053 128:1.084 256:1.376
    {4, 32},  // 16:1.280 32:1.266 64:1.290 128:1.325 256:1.678
    {16, 64},  // 16:1.905 32:1.687 64:1.655 128:1.671 256:2.063
    {256, 128},  // 16:13.926 32:8.908 64:6.529 128:5.395 256:5.890
};

}  // namespace moe355
