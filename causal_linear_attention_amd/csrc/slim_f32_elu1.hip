// Kernels for f32 I/O with the elu1 feature map.
#define SLIM_IO_T float
#define SLIM_FEAT FEAT_ELU1
#define SLIM_FEAT_IS_FAVOR 0
#define SLIM_TABLE_FN table_f32_elu1
#include "slim_inst.inc"
