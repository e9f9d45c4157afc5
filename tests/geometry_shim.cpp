// Test-only C wrappers around the product's tile-geometry header, so the CPU tests can check it
// against the oracle's mask by enumeration.
#include "../hstu_jagged_pointwise_amd/csrc/geometry.h"

extern "C" {
void shim_split(int n, int c, int t, int* nc, int* nh) { hstu::split_sequence(n, c, t, nc, nh); }
void shim_key_tiles(int rlo, int rhi, int nc, int nh, int* out3) {
    hstu::KeyTiles k = hstu::key_tiles_for_rows(rlo, rhi, nc, nh);
    out3[0] = k.main_tiles; out3[1] = k.diag_first; out3[2] = k.diag_tiles;
}
int shim_classify_row(int rlo, int rhi, int j0, int n, int nc, int nh, int keys) {
    return hstu::classify_row_tile(rlo, rhi, j0, n, nc, nh, keys);
}
void shim_rows_for_keys(int klo, int khi, int n, int nc, int nh, int* out2) {
    hstu::rows_for_keys(klo, khi, n, nc, nh, &out2[0], &out2[1]);
}
int shim_classify_key(int klo, int khi, int i0, int n, int nc, int nh, int rows) {
    return hstu::classify_key_tile(klo, khi, i0, n, nc, nh, rows);
}
int shim_ds_first_qtile(int kb, int nc) { return hstu::ds_first_qtile(kb, nc); }
int shim_ds_chunks(int kb, int n, int nc, int nh) { return hstu::ds_chunks(kb, n, nc, nh); }
long long shim_ds_chunks_before(int kb, int n, int nc, int nh) {
    return (long long)hstu::ds_chunks_before(kb, n, nc, nh);
}
}
