// host_checks.cpp -- the entry points of libmsda.so that need no GPU (the
// host validation of a level table, the workspace sizes, the status
// strings), compiled by g++ from host_checks.h: linked into libmsda.so, and
// built alone with the address and undefined-behaviour sanitizers for the
// CPU tests.  The operations are specified in include/msda.h.
#include "host_checks.h"

using namespace msda_host;

extern "C" {

msda_status msda_validate_host(const int64_t *spatial_shapes_host, const int64_t *level_start_host,
                               int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D, int64_t L,
                               int64_t K) {
    const msda_status st = check_sizes(MSDA_F32, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    return validate_levels(spatial_shapes_host, level_start_host, L, Nv, 2);
}

msda_status msda3d_validate_host(const int64_t *volume_shapes_host,
                                 const int64_t *level_start_host, int64_t B, int64_t Nv,
                                 int64_t Nq, int64_t M, int64_t D, int64_t L, int64_t K) {
    const msda_status st = check_sizes3(MSDA_F32, B, Nv, Nq, M, D, L, K);
    if (st != MSDA_OK) return st;
    return validate_levels(volume_shapes_host, level_start_host, L, Nv, 3);
}

size_t msda_backward_workspace_size(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                    int64_t L, int64_t K) {
    if (check_sizes(MSDA_F32, B, Nv, Nq, M, D, L, K) != MSDA_OK) return 0;
    if (B == 0 || Nq == 0) return 0;
    return work_layout(B, Nv, Nq, M, L, K).bytes;
}

size_t msda_backward_workspace_min(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                   int64_t L, int64_t K) {
    if (check_sizes(MSDA_F32, B, Nv, Nq, M, D, L, K) != MSDA_OK) return 0;
    if (B == 0 || Nq == 0) return 0;
    return min_workspace(Nv, Nq, L, K, false);
}

size_t msda_backward_fused_workspace_size(int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                                          int64_t D, int64_t L, int64_t K) {
    if (check_sizes(MSDA_F32, B, Nv, Nq, M, D, L, K) != MSDA_OK) return 0;
    if (B == 0 || Nq == 0) return 0;
    return fused_layout(B, Nv, Nq, M, L, K).bytes;
}

size_t msda_backward_fused_workspace_min(int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                                         int64_t D, int64_t L, int64_t K) {
    if (check_sizes(MSDA_F32, B, Nv, Nq, M, D, L, K) != MSDA_OK) return 0;
    if (B == 0 || Nq == 0) return 0;
    const FusedLayout f = fused_layout(B, Nv, Nq, M, L, K);
    return f.off_core + f.core_min;
}

size_t msda3d_backward_workspace_size(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                      int64_t L, int64_t K) {
    if (check_sizes3(MSDA_F32, B, Nv, Nq, M, D, L, K) != MSDA_OK) return 0;
    if (B == 0 || Nq == 0) return 0;
    return work_layout(B, Nv, Nq, M, L, K, true).bytes;
}

size_t msda3d_backward_workspace_min(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t D,
                                     int64_t L, int64_t K) {
    if (check_sizes3(MSDA_F32, B, Nv, Nq, M, D, L, K) != MSDA_OK) return 0;
    if (B == 0 || Nq == 0) return 0;
    return min_workspace(Nv, Nq, L, K, true);
}

const char *msda_status_string(int status) { return status_string(status); }

}  // extern "C"
