/* Plain-C use of the library's C ABI, with no GPU: the header compiles as C99, the library
 * links, and the calls that need no device (version, status strings, tiled sizes,
 * workspace sizes, argument validation) answer as documented.  Built and run by
 * tests/test_c_abi.py; prints one "name value" pair per line. */
#include <stdio.h>

#include "veda.h"

int main(void) {
  /* large workload geometry: 40 heads over a 20x48x80 latent, tile 128, three shapes */
  int32_t shapes[40][3];
  for (int h = 0; h < 40; ++h) {
    static const int32_t cyc[3][3] = {{1, 8, 16}, {2, 8, 8}, {4, 4, 8}};
    for (int a = 0; a < 3; ++a) shapes[h][a] = cyc[h % 3][a];
  }
  veda_geom g = {1, 40, 128, 20, 48, 80, 128, &shapes[0][0]};
  printf("version %s\n", veda_version());
  printf("status_null %s\n", veda_status_str(VEDA_ERR_NULL));
  printf("tiled_tokens %lld\n", (long long)veda_tiled_tokens(&g, VEDA_BF16));
  printf("head_tiles_0 %d\n", (int)veda_head_tiles(&g, VEDA_BF16, 0));
  printf("tilemap_ws_64 %zu\n", veda_oracle_tilemap_workspace_bytes(&g, 64));
  printf("trippool_ws %zu\n", veda_trippool_workspace_bytes(&g, 256, 64));
  /* validation only: each of these returns before anything is launched */
  printf("attn_null %d\n", (int)veda_sparse_attn_fwd(&g, VEDA_BF16, NULL, NULL, NULL, VEDA_TILE_COLS, NULL, NULL,
                                                      60, 0.088f, NULL, NULL, 0));
  printf("attn_dtype %d\n", (int)veda_sparse_attn_fwd(&g, (veda_dtype)7, NULL, NULL, NULL, VEDA_TILE_COLS, NULL,
                                                       NULL, 60, 0.088f, NULL, NULL, 0));
  /* a raster V has no strides in the tiled call and is refused (the fake addresses below
     are never dereferenced) */
  printf("attn_v_raster %d\n", (int)veda_sparse_attn_fwd(&g, VEDA_BF16, (const void *)256, (const void *)512,
                                                          (const void *)768, VEDA_RASTER, (const int32_t *)1024, NULL,
                                                          60, 0.088f, (void *)1280, NULL, 0));
  printf("topk_k0 %d\n", (int)veda_topk_mask(4, 10, NULL, 0, NULL, NULL, 0));
  printf("topk_empty %d\n", (int)veda_topk_mask(0, 10, (const float *)16, 3, (int32_t *)16, NULL, 0));
  int32_t bad[40][3];
  for (int h = 0; h < 40; ++h) bad[h][0] = 1, bad[h][1] = 8, bad[h][2] = 8;  /* product 64 != 128 */
  veda_geom gb = g;
  gb.tile_shapes = &bad[0][0];
  printf("tiled_tokens_bad %lld\n", (long long)veda_tiled_tokens(&gb, VEDA_BF16));
  return 0;
}
