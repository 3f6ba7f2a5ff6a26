/* A plain C caller of the library: include/convmi.h compiles as C99 and the
 * host-side entry points behave as declared, without a GPU.  Every call
 * below is a pure host query or fails validation before any launch.  Output
 * lines "key value" are checked by tests/test_c_abi.py. */
#include <stdio.h>
#include <string.h>

#include "convmi.h"

int main(void)
{
    int out = -1, rc, path = -1;

    /* Output extent: (in + 2p - d(k-1) - 1)/s + 1, and the error case. */
    rc = conv_out_size(56, 3, 2, 1, 1, &out);
    printf("out_size_56_3_2_1_1 %d %d\n", rc, out);
    rc = conv_out_size(56, 3, 1, 2, 2, &out);
    printf("out_size_56_3_1_2_2 %d %d\n", rc, out);
    rc = conv_out_size(2, 5, 1, 0, 1, &out);
    printf("out_size_too_small %d\n", rc);
    printf("last_error_set %d\n", strlen(conv_last_error()) > 0);

    /* Transposed extent: (in - 1)s - 2p + d(k - 1) + 1 + op. */
    rc = conv_transpose_out_size(28, 4, 2, 1, 1, 0, &out);
    printf("transpose_28_4_2_1_1_0 %d %d\n", rc, out);

    /* Validation before any launch: null pointers, bad groups. */
    rc = conv_fwd(NULL, NULL, NULL, NULL, 1, 8, 8, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1, 1,
                  CONV_NHWC, CONV_BF16, NULL);
    printf("fwd_null %d\n", rc);
    rc = conv_select_path(0, 1, 6, 8, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1, 4, CONV_NHWC, CONV_BF16,
                          &path);
    printf("select_bad_groups %d\n", rc);

    /* Static path selection of the five hot-path shapes. */
    rc = conv_select_path(0, 2, 3, 16, 16, 8, 3, 3, 1, 1, 1, 1, 1, 1, 1, CONV_NCHW, CONV_F32, &path);
    printf("select_tiny %d %s\n", rc, conv_path_name(path));
    rc = conv_select_path(0, 32, 256, 56, 56, 64, 1, 1, 1, 1, 0, 0, 1, 1, 1, CONV_NHWC, CONV_BF16, &path);
    printf("select_pointwise %d %s\n", rc, conv_path_name(path));
    rc = conv_select_path(0, 32, 64, 56, 56, 64, 3, 3, 1, 1, 1, 1, 1, 1, 1, CONV_NHWC, CONV_BF16, &path);
    printf("select_dense %d %s\n", rc, conv_path_name(path));
    rc = conv_select_path(0, 32, 256, 56, 56, 256, 3, 3, 1, 1, 2, 2, 2, 2, 256, CONV_NHWC, CONV_BF16,
                          &path);
    printf("select_depthwise %d %s\n", rc, conv_path_name(path));
    rc = conv_select_path(1, 32, 128, 56, 56, 256, 3, 3, 2, 2, 1, 1, 1, 1, 1, CONV_NHWC, CONV_BF16,
                          &path);
    printf("select_dx %d %s\n", rc, conv_path_name(path));
    printf("path_name_unknown %s\n", conv_path_name(12345));
    return 0;
}
