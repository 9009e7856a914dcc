/* A plain C caller of libmoe355: the host-only queries and the argument checks, which
 * touch no GPU.  Built and run by tests/test_c_abi.py with the system C compiler. */
#include <stdio.h>
#include <string.h>

#include "moe355.h"

#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                                   \
    }                                                             \
  } while (0)

int main(void) {
  /* sort buffer sizes of the DeepSeek-V3 decode layer: 64 tokens, top-8, 256 experts, M tile 16 */
  int64_t max_sorted = 0, max_blocks = 0;
  size_t ws = 0;
  EXPECT(moe_sort_sizes(64, 8, 256, 16, &max_sorted, &max_blocks, &ws) == MOE355_OK);
  EXPECT(max_sorted == 64 * 8 + 256 * 15 && max_sorted % 16 == 0);
  EXPECT(max_blocks == max_sorted / 16);
  EXPECT(moe_sort_sizes(64, 8, 256, 24, &max_sorted, NULL, NULL) == MOE355_EUNSUPPORTED);

  int bm = 0;
  EXPECT(moe_block_m(64, 8, 256, &bm) == MOE355_OK && bm == 16);
  EXPECT(moe_block_m(8192, 8, 256, &bm) == MOE355_OK && bm == 128);

  size_t bytes = 1;
  EXPECT(moe_down_combine_workspace(64, 7168, 8, &bytes) == MOE355_OK && bytes >= (size_t)64 * 8 * 7168 * 4);
  EXPECT(gemm_fp8_blockscale_workspace(4096, 18432, 7168, &bytes) == MOE355_OK && bytes == 0);
  /* the workspace follows the plan the call runs; the rule alone splits K at M = 64 */
  int tm = 0, tn = 0, sp = 0;
  EXPECT(gemm_fp8_blockscale_plan(64, 2048, 7168, 0, &tm, &tn, &sp) == MOE355_OK && sp > 1);
  EXPECT(gemm_fp8_blockscale_plan(1, 2048, 7168, 1, &tm, &tn, &sp) == MOE355_OK);
  EXPECT(gemm_fp8_blockscale_workspace(1, 2048, 7168, &bytes) == MOE355_OK &&
         bytes == (sp > 1 ? (size_t)sp * 2048 * 4 + 256 : 0));

  /* every status has a text */
  const int codes[] = {MOE355_OK, MOE355_EINVAL, MOE355_EUNSUPPORTED, MOE355_EMISALIGNED, MOE355_ELAUNCH};
  for (int i = 0; i < 5; ++i) EXPECT(moe355_strerror(codes[i]) != NULL && strlen(moe355_strerror(codes[i])) > 0);

  /* argument checks return before any launch: NULL buffers with work to do, zero tokens as a no-op */
  EXPECT(grouped_topk(NULL, 0, 256, NULL, 4, 256, 8, 4, 8, 1, 2.5f, NULL, NULL, 8, 0) == MOE355_EINVAL);
  EXPECT(grouped_topk(NULL, 0, 256, NULL, 0, 256, 8, 4, 8, 1, 2.5f, NULL, NULL, 8, 0) == MOE355_OK);
  EXPECT(fp8_quant_1x128(NULL, 7168, 0, 7168, NULL, 7168, NULL, 56, 1, 0) == MOE355_OK);
  EXPECT(gemm_fp8_blockscale(NULL, NULL, 56, 1, NULL, NULL, 0, 2048, 7168, NULL, 2048, 0, NULL, 0, 0) == MOE355_OK);
  EXPECT(gemm_fp8_blockscale(NULL, NULL, 56, 1, NULL, NULL, 4, 100, 7168, NULL, 104, 0, NULL, 0, 0) ==
         MOE355_EUNSUPPORTED);
  puts("ok");
  return 0;
}
