// device.hip -- the library's kernels as one translation unit: the
// single-launch decode kernel (single.hip) runs the bodies of the selection
// kernels (select.hip) and of the attention kernels (attend.hip), so the three
// files are compiled together here.
#include "select.hip"
#include "attend.hip"
#include "single.hip"
